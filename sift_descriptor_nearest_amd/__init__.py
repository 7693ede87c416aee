"""MI355X (gfx950) fused SIFT descriptor matcher: thin Python binding.

The C ABI in ``include/serac.h`` does all the work in HIP kernels; this
module only marshals torch CUDA tensors (device memory and the current
stream) into its arguments.  It never computes a step of the matcher
itself and has no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from collections.abc import Sequence

__all__ = ["match_pair", "match_pair_into", "match_pairs", "match_pairs_host", "top2",
           "init", "match_pair_noalloc_into", "match_pair_unfused", "match_pair_unfused_into",
           "workspace_bytes", "release_stream", "MatchLists",
           "profile_start", "profile_stop", "SeracError", "library", "LIB_PATH"]

HERE = os.path.dirname(os.path.abspath(__file__))
# SERAC_LIBRARY_PATH selects another build of the same library (the
# sanitizer tests load a host-sanitized build this way)
LIB_PATH = os.environ.get("SERAC_LIBRARY_PATH") or os.path.join(HERE, "libserac.so")
MAX_DESCRIPTORS = 262144

SERAC_OK = 0
SERAC_ERR_INVALID_ARG = -1
SERAC_ERR_CAPACITY = -2
SERAC_ERR_UNSUPPORTED_DEVICE = -3
SERAC_ERR_OUT_OF_MEMORY = -4
SERAC_ERR_HIP = -5
SERAC_ERR_TOO_LARGE = -6
SERAC_ERR_NOT_INITIALIZED = -7
SERAC_FLAG_SYMMETRIC = 1


class serac_params(ctypes.Structure):
    _fields_ = [("max_ratio", ctypes.c_double), ("max_distance", ctypes.c_double),
                ("cross_check", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("stream", ctypes.c_void_p), ("max_features", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class serac_matches(ctypes.Structure):
    _fields_ = [("matches", ctypes.c_void_p), ("capacity", ctypes.c_int64),
                ("count", ctypes.c_void_p)]


class serac_pair(ctypes.Structure):
    _fields_ = [("a", ctypes.c_int32), ("b", ctypes.c_int32)]


class SeracError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {library().serac_status_string(status).decode()} "
                         f"(status {status})")


_lib = None


def library(path: str = LIB_PATH) -> ctypes.CDLL:
    """The loaded C ABI.  Raises if the library has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is missing: build it with "
                           "__graft_entry__.build() (hipcc, gfx950)")
    L = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    L.serac_match_pair.argtypes = [vp, i32, vp, i32, ctypes.POINTER(serac_params),
                                   ctypes.POINTER(serac_matches)]
    L.serac_match_pairs.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(i32), i32,
                                    ctypes.POINTER(serac_pair), i32,
                                    ctypes.POINTER(serac_params),
                                    ctypes.POINTER(serac_matches)]
    L.serac_match_pairs_host.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(i32), i32,
                                         ctypes.POINTER(serac_pair), i32,
                                         ctypes.POINTER(serac_params), i32,
                                         ctypes.POINTER(vp), ctypes.POINTER(i32)]
    L.serac_match_pair_noalloc.argtypes = L.serac_match_pair.argtypes
    L.serac_init.argtypes = []
    L.serac_match_pair_unfused.argtypes = L.serac_match_pair.argtypes
    L.serac_workspace_bytes.argtypes = [ctypes.POINTER(ctypes.c_int64)]
    L.serac_release_stream.argtypes = [vp]
    L.serac_top2_pair.argtypes = [vp, i32, vp, i32, vp, vp, vp]
    L.serac_profile_start.argtypes = [i32, i32]
    L.serac_profile_stop.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32),
                                     ctypes.POINTER(ctypes.c_float), i32,
                                     ctypes.POINTER(ctypes.c_char_p)]
    L.serac_angle_slack.argtypes = [ctypes.POINTER(ctypes.c_double)]
    L.serac_angle_slack.restype = ctypes.c_int
    L.serac_status_string.argtypes = [ctypes.c_int]
    L.serac_status_string.restype = ctypes.c_char_p
    for f in (L.serac_match_pair, L.serac_match_pairs, L.serac_match_pairs_host,
              L.serac_top2_pair, L.serac_init, L.serac_match_pair_noalloc,
              L.serac_match_pair_unfused, L.serac_workspace_bytes, L.serac_release_stream,
              L.serac_profile_start, L.serac_profile_stop):
        f.restype = ctypes.c_int
    _lib = L
    return L


def _check_desc(x, name):
    import torch
    if not isinstance(x, torch.Tensor) or x.dtype != torch.uint8 or x.dim() != 2 \
            or x.shape[1] != 128 or not x.is_cuda or not x.is_contiguous():
        raise ValueError(f"{name} must be a contiguous torch.uint8 CUDA tensor [n, 128]")
    if x.shape[0] > MAX_DESCRIPTORS:
        raise ValueError(f"{name} has more than {MAX_DESCRIPTORS} descriptors")
    if x.shape[0] and x.data_ptr() % 16:
        raise ValueError(f"{name} must start on a 16-byte boundary (the kernels read "
                         "16-byte words); a view at an odd storage offset does not")


def _check_out(out, count, nA, device):
    """out: int32 [>= nA, 2], count: int32 [>= 1], contiguous, on `device`."""
    import torch
    for t, name in ((out, "out"), (count, "count")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or not t.is_cuda \
                or not t.is_contiguous() or t.device != device:
            raise ValueError(f"{name} must be a contiguous torch.int32 tensor on {device}")
    if out.dim() != 2 or out.shape[1] != 2 or out.shape[0] < nA:
        raise ValueError(f"out must have shape [>= {nA}, 2], got {list(out.shape)}")
    if count.numel() < 1:
        raise ValueError("count must hold at least one int32")
    if (nA and out.data_ptr() % 8) or count.data_ptr() % 4:
        raise ValueError("out must be 8-byte aligned and count 4-byte aligned")


def _params(max_ratio, max_distance, cross_check, stream, symmetric=False, max_features=0):
    return serac_params(float(max_ratio), float(max_distance), int(bool(cross_check)),
                        SERAC_FLAG_SYMMETRIC if symmetric else 0, ctypes.c_void_p(stream),
                        int(max_features), 0)


def _capped(n, max_features):
    return min(n, max_features) if max_features > 0 else n


def _stream(device):
    """The raw hipStream_t of torch's current stream on `device`.  torch's
    internal accessor returns it directly (~0.2 us); building the public
    Stream object costs ~2 us per call, a sixth of an 8192 x 8192 call's
    host time."""
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(device.index if device.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


def match_pair_into(a, b, out, count, max_ratio=0.8, max_distance=math.inf,
                    cross_check=True, stream=None, symmetric=False, max_features=0) -> None:
    """Enqueue one pair; out is int32 [>= nA, 2], count int32 [1] (device).

    Asynchronous on the current stream (or ``stream``, a raw hipStream_t);
    nothing is synchronised.  symmetric: the column side passes the same
    gates (SERAC_FLAG_SYMMETRIC); max_features: the match cap (only the
    first max_features rows of each set take part; 0 = none).
    """
    _check_desc(a, "a")
    _check_desc(b, "b")
    if b.device != a.device:
        raise ValueError("a and b must be on the same device")
    _check_out(out, count, _capped(a.shape[0], max_features), a.device)
    s = _stream(a.device) if stream is None else stream
    p = _params(max_ratio, max_distance, cross_check, s, symmetric, max_features)
    m = serac_matches(out.data_ptr(), out.shape[0], count.data_ptr())
    rc = library().serac_match_pair(a.data_ptr(), a.shape[0], b.data_ptr(), b.shape[0],
                                    ctypes.byref(p), ctypes.byref(m))
    if rc != SERAC_OK:
        raise SeracError(rc, "serac_match_pair")


def init(device=None) -> None:
    """Set up `device` (default: the current one) for the library: what the
    first call of any entry point on it would do, including the fixed
    scratch of serac_match_pair_noalloc."""
    import torch
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        rc = library().serac_init()
    if rc != SERAC_OK:
        raise SeracError(rc, "serac_init")


def match_pair_noalloc_into(a, b, out, count, max_ratio=0.8, max_distance=math.inf,
                            cross_check=True, stream=None, max_features=0) -> None:
    """match_pair_into through serac_match_pair_noalloc: no device
    allocation inside the library (the device must have been set up, e.g.
    by init()).  Calls that overlap on one device race."""
    _check_desc(a, "a")
    _check_desc(b, "b")
    if b.device != a.device:
        raise ValueError("a and b must be on the same device")
    _check_out(out, count, _capped(a.shape[0], max_features), a.device)
    s = _stream(a.device) if stream is None else stream
    p = _params(max_ratio, max_distance, cross_check, s, False, max_features)
    m = serac_matches(out.data_ptr(), out.shape[0], count.data_ptr())
    rc = library().serac_match_pair_noalloc(a.data_ptr(), a.shape[0], b.data_ptr(),
                                            b.shape[0], ctypes.byref(p), ctypes.byref(m))
    if rc != SERAC_OK:
        raise SeracError(rc, "serac_match_pair_noalloc")


def match_pair(a, b, max_ratio=0.8, max_distance=math.inf, cross_check=True,
               symmetric=False, max_features=0):
    """Matches of one pair as int32 [count, 2] = (row of a, row of b).

    Synchronises the stream to read the count.
    """
    import torch
    out = torch.empty((max(a.shape[0], 1), 2), dtype=torch.int32, device=a.device)
    count = torch.empty(1, dtype=torch.int32, device=a.device)
    match_pair_into(a, b, out, count, max_ratio, max_distance, cross_check,
                    symmetric=symmetric, max_features=max_features)
    n = int(count.item())
    if n < 0:
        raise SeracError(SERAC_ERR_HIP, "serac_match_pair: ordered output hand-off failed")
    return out[:n]


def match_pair_unfused_into(a, b, out, count, max_ratio=0.8, max_distance=math.inf,
                            cross_check=True, stream=None, max_features=0) -> None:
    """match_pair_into through the unfused arm (serac_match_pair_unfused:
    the score matrix written to device memory, then row and column passes).
    Same result; for comparison.  Asynchronous like match_pair_into."""
    _check_desc(a, "a")
    _check_desc(b, "b")
    if b.device != a.device:
        raise ValueError("a and b must be on the same device")
    _check_out(out, count, _capped(a.shape[0], max_features), a.device)
    s = _stream(a.device) if stream is None else stream
    p = _params(max_ratio, max_distance, cross_check, s, False, max_features)
    m = serac_matches(out.data_ptr(), out.shape[0], count.data_ptr())
    rc = library().serac_match_pair_unfused(a.data_ptr(), a.shape[0], b.data_ptr(), b.shape[0],
                                            ctypes.byref(p), ctypes.byref(m))
    if rc != SERAC_OK:
        raise SeracError(rc, "serac_match_pair_unfused")


def match_pair_unfused(a, b, max_ratio=0.8, max_distance=math.inf, cross_check=True,
                       max_features=0):
    """The list of match_pair_unfused_into as int32 [count, 2]; synchronises
    the stream."""
    import torch
    out = torch.empty((max(a.shape[0], 1), 2), dtype=torch.int32, device=a.device)
    count = torch.empty(1, dtype=torch.int32, device=a.device)
    match_pair_unfused_into(a, b, out, count, max_ratio, max_distance, cross_check,
                            max_features=max_features)
    n = int(count.item())
    if n < 0:
        raise SeracError(SERAC_ERR_HIP, "serac_match_pair_unfused: ordered output hand-off failed")
    return out[:n]


def release_stream(stream=None, device=None) -> None:
    """Free the library's workspace for a stream (default: torch's current
    stream on `device`); a later call on it allocates a new one."""
    import torch
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    s = _stream(dev) if stream is None else stream
    rc = library().serac_release_stream(ctypes.c_void_p(s))
    if rc != SERAC_OK:
        raise SeracError(rc, "serac_release_stream")


def workspace_bytes() -> int:
    """Device bytes the library's workspaces hold on the current device."""
    v = ctypes.c_int64(0)
    rc = library().serac_workspace_bytes(ctypes.byref(v))
    if rc != SERAC_OK:
        raise SeracError(rc, "serac_workspace_bytes")
    return v.value


class MatchLists(Sequence):
    """The match lists of a batch, one per pair in pair order: a read-only
    sequence whose item q is a view of the rows [offset q, + count q) of one
    buffer (a torch tensor for match_pairs, a numpy array for
    match_pairs_host).  Views are made when an item is read (~2 us each),
    so a call over many pairs does not build them all up front (for 1128
    pairs that took ~2 ms, a sixth of the call's time)."""

    __slots__ = ("_buf", "_offs", "_cnt")

    def __init__(self, buf, offs, counts):
        self._buf = buf
        self._offs = [int(x) for x in offs] if not hasattr(offs, "tolist") else offs.tolist()
        self._cnt = [int(x) for x in counts] if not hasattr(counts, "tolist") else counts.tolist()

    def __len__(self):
        return len(self._cnt)

    def __getitem__(self, q):
        if isinstance(q, slice):
            return [self[k] for k in range(*q.indices(len(self)))]
        q = int(q)
        if q < 0:
            q += len(self)
        if not 0 <= q < len(self):
            raise IndexError("pair index out of range")
        o = self._offs[q]
        return self._buf[o:o + self._cnt[q]]


def match_pairs(images, pairs, max_ratio=0.8, max_distance=math.inf,
                cross_check=True, symmetric=False, max_features=0):
    """Match many pairs of one image set in one call.

    images: list of uint8 CUDA tensors [n_k, 128] on one device;
    pairs: sequence of (a, b) image indices.  Returns a MatchLists of int32
    [count, 2] tensors (views of one device buffer), one per pair, in order.
    """
    import torch
    for k, x in enumerate(images):
        _check_desc(x, f"images[{k}]")
        if x.device != images[0].device:
            raise ValueError("all images must be on one device")
    import numpy as np
    pr = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    P = pr.shape[0]
    if P == 0:
        return []
    dev = images[0].device
    nimg = np.array([x.shape[0] for x in images], dtype=np.int64)
    if pr.min() < 0 or pr.max() >= len(images):
        raise SeracError(SERAC_ERR_INVALID_ARG, "serac_match_pairs")
    caps = np.maximum(nimg[pr[:, 0]], 1)
    offs = np.zeros(P + 1, dtype=np.int64)
    np.cumsum(caps, out=offs[1:])
    out = torch.empty((int(offs[-1]), 2), dtype=torch.int32, device=dev)
    counts = torch.empty(P, dtype=torch.int32, device=dev)
    ptrs = (ctypes.c_void_p * len(images))(*[x.data_ptr() for x in images])
    ns = nimg.astype(np.int32)
    cp = np.ascontiguousarray(pr.astype(np.int32))          # serac_pair [P]
    ms = np.zeros(P, dtype=[("matches", np.uint64), ("capacity", np.int64),
                            ("count", np.uint64)])          # serac_matches [P]
    ms["matches"] = out.data_ptr() + offs[:-1] * 8
    ms["capacity"] = caps
    ms["count"] = counts.data_ptr() + 4 * np.arange(P, dtype=np.uint64)
    prm = _params(max_ratio, max_distance, cross_check, _stream(dev), symmetric, max_features)
    rc = library().serac_match_pairs(ptrs, ns.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                     len(images), cp.ctypes.data_as(ctypes.POINTER(serac_pair)),
                                     P, ctypes.byref(prm),
                                     ms.ctypes.data_as(ctypes.POINTER(serac_matches)))
    if rc != SERAC_OK:
        raise SeracError(rc, "serac_match_pairs")
    cnt = counts.cpu().numpy().astype(np.int64)
    if cnt.min() < 0:
        raise SeracError(SERAC_ERR_HIP, "serac_match_pairs: ordered output hand-off failed")
    return MatchLists(out, offs, cnt)


def match_pairs_host(images, pairs, max_ratio=0.8, max_distance=math.inf,
                     cross_check=True, pairs_per_stage=0, symmetric=False, max_features=0):
    """Match many pairs and return the match lists in host memory.

    Same inputs and results as match_pairs, but the lists arrive as numpy
    uint32 [count, 2] arrays: the library overlaps copying finished stages
    to the host with matching the next ones (serac_match_pairs_host).
    Returns when every list is on the host.
    """
    import numpy as np
    for k, x in enumerate(images):
        _check_desc(x, f"images[{k}]")
        if x.device != images[0].device:
            raise ValueError("all images must be on one device")
    pr = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    P = pr.shape[0]
    if P == 0:
        return []
    if pr.min() < 0 or pr.max() >= len(images):
        raise SeracError(SERAC_ERR_INVALID_ARG, "serac_match_pairs_host")
    nimg = np.array([x.shape[0] for x in images], dtype=np.int64)
    caps = nimg[pr[:, 0]]
    offs = np.zeros(P + 1, dtype=np.int64)
    np.cumsum(caps, out=offs[1:])
    host = np.empty((max(int(offs[-1]), 1), 2), dtype=np.uint32)
    counts = np.empty(P, dtype=np.int32)
    ptrs = (ctypes.c_void_p * len(images))(*[x.data_ptr() for x in images])
    ns = nimg.astype(np.int32)
    cp = np.ascontiguousarray(pr.astype(np.int32))          # serac_pair [P]
    hp = (host.ctypes.data + offs[:-1] * 8).astype(np.uint64)
    prm = _params(max_ratio, max_distance, cross_check, _stream(images[0].device), symmetric,
                  max_features)
    rc = library().serac_match_pairs_host(
        ptrs, ns.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(images),
        cp.ctypes.data_as(ctypes.POINTER(serac_pair)), P, ctypes.byref(prm),
        int(pairs_per_stage), hp.ctypes.data_as(ctypes.POINTER(ctypes.c_void_p)),
        counts.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    if rc != SERAC_OK:
        raise SeracError(rc, "serac_match_pairs_host")
    if counts.min() < 0:
        raise SeracError(SERAC_ERR_HIP, "serac_match_pairs_host: ordered output hand-off failed")
    return MatchLists(host, offs, counts)


def top2(a, b):
    """(row_top2 int32 [nA, 3] = best, idx, second; col_best int32 [nB, 2])."""
    import torch
    _check_desc(a, "a")
    _check_desc(b, "b")
    if b.device != a.device:
        raise ValueError("a and b must be on the same device")
    row = torch.empty((a.shape[0], 3), dtype=torch.int32, device=a.device)
    col = torch.empty((b.shape[0], 2), dtype=torch.int32, device=a.device)
    rc = library().serac_top2_pair(a.data_ptr(), a.shape[0], b.data_ptr(), b.shape[0],
                                   ctypes.c_void_p(_stream(a.device)),
                                   row.data_ptr() if a.shape[0] else None,
                                   col.data_ptr() if b.shape[0] else None)
    if rc != SERAC_OK:
        raise SeracError(rc, "serac_top2_pair")
    return row, col


def profile_start(max_launches: int, every: int = 1) -> None:
    """Time up to max_launches of the following tile-kernel launches, one in
    `every`, with HIP events attached to their dispatches."""
    rc = library().serac_profile_start(int(max_launches), int(every))
    if rc != SERAC_OK:
        raise SeracError(rc, "serac_profile_start")


def profile_stop(capacity: int = 1 << 16):
    """(summed tile-kernel device ms, launches timed, per-launch ms list,
    name of the tile kernel timed); disarms."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int32(0)
    per = (ctypes.c_float * max(capacity, 1))()
    name = ctypes.c_char_p()
    rc = library().serac_profile_stop(ctypes.byref(ms), ctypes.byref(n), per, int(capacity),
                                      ctypes.byref(name))
    if rc != SERAC_OK:
        raise SeracError(rc, "serac_profile_stop")
    return ms.value, n.value, list(per[:min(n.value, capacity)]), name.value.decode()


def angle_slack() -> float:
    """Half-width of the interval around the device angle inside which the
    finishing kernel trusts it (inf: the table decides every gate)."""
    v = ctypes.c_double(0.0)
    rc = library().serac_angle_slack(ctypes.byref(v))
    if rc != SERAC_OK:
        raise SeracError(rc, "serac_angle_slack")
    return v.value


PROBE_PATH = os.path.join(HERE, "libserac_probe.so")
_probe = None


def probe_mfma(blocks: int, iters: int, nv: int = 0):
    """Back-to-back int8 MFMA rate with nv vector instructions per MFMA
    (libserac_probe.so): (device ms, TOPS, shader clock GHz)."""
    global _probe
    if _probe is None:
        if not os.path.exists(PROBE_PATH):
            raise RuntimeError(f"{PROBE_PATH} is missing: build it with __graft_entry__.build()")
        P = ctypes.CDLL(PROBE_PATH)
        d = ctypes.POINTER(ctypes.c_double)
        P.serac_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, d, d, d]
        P.serac_probe_mfma.restype = ctypes.c_int
        _probe = P
    ms, tops, ghz = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    rc = _probe.serac_probe_mfma(int(blocks), int(iters), int(nv), ctypes.byref(ms),
                                 ctypes.byref(tops), ctypes.byref(ghz))
    if rc != 0:
        raise RuntimeError(f"serac_probe_mfma failed ({rc})")
    return ms.value, tops.value, ghz.value
