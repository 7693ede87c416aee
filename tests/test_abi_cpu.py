"""The C ABI on the CPU: it loads, exports what the header declares, and
rejects bad arguments before touching HIP (no compute call is made)."""
import ctypes
import math
import os
import re

import pytest

import sift_descriptor_nearest_amd as serac
from sift_descriptor_nearest_amd import serac_matches, serac_pair, serac_params

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "serac.h")
FAKE = 0x10000          # never dereferenced: validation fails first


def declared(header=HEADER):
    src = open(header).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(serac_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    L = serac.library()
    names = declared() + declared(os.path.join(ROOT, "include", "serac_bench.h"))
    assert {"serac_match_pair", "serac_match_pairs", "serac_top2_pair",
            "serac_init", "serac_match_pair_noalloc", "serac_match_pair_unfused",
            "serac_workspace_bytes", "serac_status_string", "serac_profile_start", "serac_profile_stop",
            "serac_angle_slack"} <= set(names)
    for name in names:
        assert hasattr(L, name), name


def test_probe_library_exports_its_header():
    P = ctypes.CDLL(serac.PROBE_PATH)
    names = declared(os.path.join(ROOT, "include", "serac_probe.h"))
    assert names == ["serac_probe_mfma"]
    for name in names:
        assert hasattr(P, name), name


def test_every_header_is_checked():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == \
        ["serac.h", "serac_bench.h", "serac_probe.h"]


def test_status_strings():
    L = serac.library()
    for st in (0, -1, -2, -3, -4, -5, -6, -7):
        assert L.serac_status_string(st)
    assert L.serac_status_string(12345) == b"unknown status"


def _p(**kw):
    d = dict(max_ratio=0.8, max_distance=math.inf, cross_check=1, flags=0, stream=None,
             max_features=0, reserved=0)
    d.update(kw)
    return serac_params(d["max_ratio"], d["max_distance"], d["cross_check"], d["flags"],
                        d["stream"], d["max_features"], d["reserved"])


def _m(cap=100):
    return serac_matches(FAKE, cap, FAKE)


def call_pair(a=FAKE, nA=10, b=FAKE, nB=10, params="ok", out="ok"):
    L = serac.library()
    pp = ctypes.byref(_p()) if params == "ok" else params
    oo = ctypes.byref(_m()) if out == "ok" else out
    return L.serac_match_pair(a, nA, b, nB, pp, oo)


BAD_PARAMS = [
    dict(max_ratio=float("nan")), dict(max_ratio=0.0), dict(max_ratio=-1.0),
    dict(max_ratio=math.inf), dict(max_distance=float("nan")),
    dict(max_distance=-0.1), dict(cross_check=2), dict(cross_check=-1), dict(flags=2),
    dict(flags=-1), dict(flags=3), dict(max_features=-1), dict(reserved=1),
]


@pytest.mark.parametrize("kw", BAD_PARAMS, ids=[str(k) for k in BAD_PARAMS])
def test_match_pair_rejects_bad_params(kw):
    assert call_pair(params=ctypes.byref(_p(**kw))) == serac.SERAC_ERR_INVALID_ARG


def test_match_pair_rejects_bad_sets():
    E = serac.SERAC_ERR_INVALID_ARG
    assert call_pair(a=None) == E
    assert call_pair(b=None) == E
    assert call_pair(nA=-1) == E
    assert call_pair(nB=-5) == E
    assert call_pair(nA=serac.MAX_DESCRIPTORS + 1) == E
    assert call_pair(params=None) == E
    assert call_pair(out=None) == E
    assert call_pair(out=ctypes.byref(serac_matches(None, 100, FAKE))) == E
    assert call_pair(out=ctypes.byref(serac_matches(FAKE, 100, None))) == E


def test_match_pair_rejects_misaligned_pointers():
    """Descriptors must be 16-byte aligned, match arrays 8, counts 4."""
    E = serac.SERAC_ERR_INVALID_ARG
    assert call_pair(a=FAKE + 8) == E
    assert call_pair(b=FAKE + 1) == E
    assert call_pair(out=ctypes.byref(serac_matches(FAKE + 4, 100, FAKE))) == E
    assert call_pair(out=ctypes.byref(serac_matches(FAKE, 100, FAKE + 2))) == E
    L = serac.library()
    assert L.serac_top2_pair(FAKE, 3, FAKE, 3, None, FAKE + 2, FAKE) == E
    assert L.serac_top2_pair(FAKE, 3, FAKE, 3, None, FAKE, FAKE + 1) == E


def test_match_pair_noalloc_validation():
    """The non-allocating entry point validates as serac_match_pair does and
    refuses, before any HIP call, a pair beyond its single-kernel limit."""
    L = serac.library()
    E = serac.SERAC_ERR_INVALID_ARG

    def call(a=FAKE, nA=10, b=FAKE, nB=10, params=None, out=None):
        pp = ctypes.byref(params or _p())
        oo = ctypes.byref(out or _m())
        return L.serac_match_pair_noalloc(a, nA, b, nB, pp, oo)

    assert call(a=None) == E
    assert call(b=FAKE + 8) == E
    assert call(nA=-1) == E
    assert call(params=_p(flags=1)) == E
    assert call(params=_p(max_ratio=0.0)) == E
    assert call(params=_p(flags=serac.SERAC_FLAG_SYMMETRIC)) == E     # not on this path
    assert call(params=_p(max_features=-3)) == E
    assert call(out=serac_matches(FAKE + 4, 100, FAKE)) == E
    assert L.serac_match_pair_noalloc(FAKE, 10, FAKE, 10, None, ctypes.byref(_m())) == E
    assert L.serac_match_pair_noalloc(FAKE, 10, FAKE, 10, ctypes.byref(_p()), None) == E
    assert call(nA=101) == serac.SERAC_ERR_CAPACITY
    big = serac_matches(FAKE, 1 << 20, FAKE)
    assert call(nA=16385, nB=16385, out=big) == serac.SERAC_ERR_TOO_LARGE
    assert call(nA=1, nB=(1 << 28) + 1, out=big) == serac.SERAC_ERR_INVALID_ARG   # > max set
    assert call(nA=2048, nB=131073, out=big) == serac.SERAC_ERR_TOO_LARGE


def test_match_pair_unfused_validation():
    L = serac.library()
    E = serac.SERAC_ERR_INVALID_ARG

    def call(a=FAKE, nA=10, b=FAKE, nB=10, params=None, out=None):
        return L.serac_match_pair_unfused(a, nA, b, nB, ctypes.byref(params or _p()),
                                          ctypes.byref(out or _m()))

    assert call(a=None) == E
    assert call(b=FAKE + 4) == E
    assert call(params=_p(flags=serac.SERAC_FLAG_SYMMETRIC)) == E
    assert call(params=_p(cross_check=3)) == E
    assert call(nA=101) == serac.SERAC_ERR_CAPACITY
    big = serac_matches(FAKE, 1 << 20, FAKE)
    assert call(nA=65537, nB=65537, out=big) == serac.SERAC_ERR_TOO_LARGE
    assert L.serac_workspace_bytes(None) == E


def test_match_pair_rejects_small_capacity():
    assert call_pair(nA=101) == serac.SERAC_ERR_CAPACITY
    assert call_pair(nA=10, out=ctypes.byref(_m(9))) == serac.SERAC_ERR_CAPACITY
    # under a match cap the capacity needed is min(nA, max_features)
    capped = ctypes.byref(_p(max_features=150))
    assert call_pair(nA=200, params=capped) == serac.SERAC_ERR_CAPACITY
    assert call_pair(nA=200, params=capped, out=ctypes.byref(_m(149))) == \
        serac.SERAC_ERR_CAPACITY


def test_params_layout():
    """The binding's structure has the header's layout (x86-64)."""
    assert ctypes.sizeof(serac_params) == 40
    assert serac_params.stream.offset == 24
    assert serac_params.max_features.offset == 32
    assert serac_params.reserved.offset == 36


def test_match_pairs_validation():
    L = serac.library()
    ptrs = (ctypes.c_void_p * 2)(FAKE, FAKE)
    ns = (ctypes.c_int32 * 2)(10, 20)
    ok = ctypes.byref(_p())

    def run(pairs, outs, ns=ns, num_images=2, params=ok):
        cp = (serac_pair * len(pairs))(*[serac_pair(*p) for p in pairs])
        ms = (serac_matches * len(outs))(*outs)
        return L.serac_match_pairs(ptrs, ns, num_images, cp, len(pairs), params, ms)

    E = serac.SERAC_ERR_INVALID_ARG
    assert run([(0, 2)], [_m()]) == E                     # image index out of range
    assert run([(-1, 1)], [_m()]) == E
    assert run([(0, 1)], [_m()], params=ctypes.byref(_p(flags=3))) == E
    assert run([(1, 0)], [_m(19)]) == serac.SERAC_ERR_CAPACITY
    assert run([(0, 1)], [serac_matches(FAKE, 100, None)]) == E
    assert run([(0, 1)], [serac_matches(FAKE + 4, 100, FAKE)]) == E   # misaligned list
    bad_ptrs = (ctypes.c_void_p * 2)(FAKE, FAKE + 16 + 8)             # misaligned image
    cp = (serac_pair * 1)(serac_pair(0, 1))
    ms = (serac_matches * 1)(_m())
    assert L.serac_match_pairs(bad_ptrs, ns, 2, cp, 1, ok, ms) == E
    bad_n = (ctypes.c_int32 * 2)(10, -1)
    assert run([(0, 1)], [_m()], ns=bad_n) == E
    assert L.serac_match_pairs(ptrs, ns, -1, None, 0, ok, None) == E
    # no pairs: nothing to do, nothing touched
    assert L.serac_match_pairs(None, None, 0, None, 0, ok, None) == serac.SERAC_OK


def test_match_pairs_host_validation():
    L = serac.library()
    ptrs = (ctypes.c_void_p * 2)(FAKE, FAKE)
    ns = (ctypes.c_int32 * 2)(10, 0)
    ok = ctypes.byref(_p())
    counts = (ctypes.c_int32 * 4)()

    def run(pairs, hosts, ns=ns, num_images=2, params=ok, per=0, counts=counts):
        cp = (serac_pair * len(pairs))(*[serac_pair(*p) for p in pairs])
        hp = (ctypes.c_void_p * len(hosts))(*hosts)
        return L.serac_match_pairs_host(ptrs, ns, num_images, cp, len(pairs), params, per, hp,
                                        counts)

    E = serac.SERAC_ERR_INVALID_ARG
    assert run([(0, 2)], [FAKE]) == E                     # image index out of range
    assert run([(0, 1)], [FAKE], per=-1) == E             # stage size
    assert run([(0, 1)], [None]) == E                     # no host array for 10 matches
    assert run([(0, 1)], [FAKE], counts=None) == E
    assert run([(0, 1)], [FAKE], params=ctypes.byref(_p(max_ratio=0.0))) == E
    assert run([(0, 1)], [FAKE], ns=(ctypes.c_int32 * 2)(-1, 3)) == E
    assert L.serac_match_pairs_host(ptrs, ns, 2, None, 1, ok, 0, None, counts) == E
    # no pairs: nothing to do, nothing touched
    assert L.serac_match_pairs_host(None, None, 0, None, 0, ok, 0, None, None) == serac.SERAC_OK


def test_top2_validation():
    L = serac.library()
    E = serac.SERAC_ERR_INVALID_ARG
    assert L.serac_top2_pair(None, 3, FAKE, 3, None, FAKE, FAKE) == E
    assert L.serac_top2_pair(FAKE, 3, FAKE, 3, None, None, FAKE) == E
    assert L.serac_top2_pair(FAKE, 3, FAKE, 3, None, FAKE, None) == E
    assert L.serac_top2_pair(FAKE, -3, FAKE, 3, None, FAKE, FAKE) == E


def test_binding_rejects_non_tensors():
    with pytest.raises(ValueError):
        serac.match_pair_into(object(), object(), None, None)


def test_binding_checks_outputs_and_alignment():
    """The binding's own checks run before any device work, so they can be
    exercised with CPU tensors standing in for device ones (is_cuda is
    patched on the stand-ins)."""
    import torch

    class Fake(torch.Tensor):
        @property
        def is_cuda(self):
            return True

    def fake(t):
        return t.as_subclass(Fake)

    a = fake(torch.zeros((4, 128), dtype=torch.uint8))
    b = fake(torch.zeros((5, 128), dtype=torch.uint8))
    out = fake(torch.zeros((4, 2), dtype=torch.int32))
    cnt = fake(torch.zeros(1, dtype=torch.int32))
    bad = [
        (fake(torch.zeros((4, 2), dtype=torch.int16)), cnt),      # dtype
        (fake(torch.zeros(8, dtype=torch.int32)), cnt),           # 1-D
        (fake(torch.zeros((3, 2), dtype=torch.int32)), cnt),      # too few rows
        (fake(torch.zeros((4, 4), dtype=torch.int32)[:, :2]), cnt),   # not contiguous
        (out, fake(torch.zeros(0, dtype=torch.int32))),           # empty count
        (out, fake(torch.zeros(1, dtype=torch.int64))),           # count dtype
        (out, torch.zeros(1, dtype=torch.int32)),                 # count not on the device
    ]
    for o, c in bad:
        with pytest.raises(ValueError):
            serac.match_pair_into(a, b, o, c)
    # a descriptor view at an odd storage offset is not 16-byte aligned
    storage = torch.zeros(5 * 128 + 16, dtype=torch.uint8)
    shift = 8 if storage.data_ptr() % 16 == 0 else 16 - storage.data_ptr() % 16 + 8
    odd = fake(storage[shift:shift + 4 * 128].view(4, 128))
    assert odd.data_ptr() % 16 == 8
    with pytest.raises(ValueError):
        serac.match_pair_into(odd, b, out, cnt)
