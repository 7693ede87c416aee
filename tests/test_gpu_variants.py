"""The parameter variants on the HIP path against the CPU oracle, through the
C ABI: symmetric column gates (SERAC_FLAG_SYMMETRIC) and the match cap
(max_features), alone and together, for one pair and for batches.

Lists must be byte-identical to the oracle's.  Above the sizes the oracle
finishes in seconds, the symmetric list is checked against a property that
holds at any size: it is the cross-checked list of (A, B) intersected with
the transposed cross-checked list of (B, A), both from the library's own
(parity-tested) default path.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from oracle_pins import tie_heavy
from sift_descriptor_nearest_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def serac():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sift_descriptor_nearest_amd as s
    s.library()
    return s


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def check(serac, A, B, r=0.8, d=math.inf, c=True, sym=False, cap=0, label=""):
    say(f"[variants] {label} nA={len(A)} nB={len(B)} ratio={r} dist={d} cross={c} "
        f"sym={sym} cap={cap}")
    got = serac.match_pair(dev(A), dev(B), r, d, c, symmetric=sym, max_features=cap)
    got = got.cpu().numpy().astype(np.uint32)
    want = oracle.match_pair(A, B, r, d, c, symmetric=sym, max_features=cap)
    assert got.shape == want.shape, (label, got.shape, want.shape)
    assert got.tobytes() == want.tobytes(), label
    return got


SMALL = [(1, 1), (3, 700), (700, 3), (255, 257), (513, 300), (1029, 777)]


def tie_heavy_no255(rng, n):
    """tie_heavy rows without its all-255 rows (one such column is every
    row's best and leaves nothing to match)."""
    X = tie_heavy(rng, n)
    X[(X == 255).all(axis=1)] = 0
    return X


@pytest.mark.parametrize("nA,nB", SMALL, ids=[f"{a}x{b}" for a, b in SMALL])
def test_symmetric_tie_heavy(serac, nA, nB):
    """Planted edge pairs with a quarter of tie-heavy rows on each side, and
    tie-heavy pairs (where the column gate removes mutual matches at ratio
    1.0), at strict and lenient ratios."""
    rng = np.random.default_rng(nA * 7919 + nB)
    p = synth.edge_pair(nA, nB, max(1, min(nA, nB) // 3), min(nA, nB) // 10, False, nA + nB)
    A, B = p.A.copy(), p.B.copy()
    if nA // 4:
        A[-(nA // 4):] = tie_heavy_no255(rng, nA // 4)
    if nB // 4:
        B[-(nB // 4):] = tie_heavy_no255(rng, nB // 4)
    T, U = tie_heavy_no255(rng, nA), tie_heavy_no255(rng, nB)
    for r, d in ((0.8, math.inf), (1.0, math.inf), (1.3, math.inf), (1.3, 1.2)):
        check(serac, A, B, r, d, True, True, label="planted + tie-heavy")
        check(serac, T, U, r, d, True, True, label="tie-heavy")


@pytest.mark.parametrize("k", range(12))
def test_symmetric_random(serac, k):
    rng = np.random.default_rng(1000 + k)
    nA = int(rng.integers(1, 3000))
    nB = int(rng.integers(1, 3000))
    kind = k % 3
    if kind == 0:
        p = synth.pair(nA, nB, float(rng.uniform(0.05, 0.5)), int(rng.integers(1, 12)), k)
        A, B = p.A, p.B
    elif kind == 1:
        p = synth.edge_pair(nA, nB, min(nA, nB) // 4, min(nA, nB) // 20, bool(k & 1), k)
        A, B = p.A, p.B
    else:
        A, B = tie_heavy(rng, nA), tie_heavy(rng, nB)
    r = float(rng.choice([0.6, 0.8, 0.95, 1.2]))
    # (tie-heavy rows score low: their angles pass no finite distance gate)
    d = math.inf if kind == 2 else float(rng.choice([0.7, math.inf]))
    check(serac, A, B, r, d, bool(k & 2), True, label=f"random {k}")


def test_symmetric_workload_8192(serac):
    p = synth.workload("pair_8192x8192")
    got = check(serac, p.A, p.B, 0.8, 0.7, True, True, label="pair_8192x8192")
    cross = oracle.match_pair(p.A, p.B, 0.8, 0.7, True)
    assert 0 < len(got) <= len(cross)


def test_symmetric_empty_sides(serac):
    e = np.zeros((0, 128), np.uint8)
    x = synth.pair(300, 10, 0.2, 4, seed=2).A
    for A, B in ((e, x), (x, e)):
        got = serac.match_pair(dev(A), dev(B), symmetric=True)
        assert got.shape == (0, 2)


def _set(got):
    return {tuple(t) for t in got.cpu().numpy().tolist()}


@pytest.mark.parametrize("nA,nB", [(16385, 16384), (8192, 32769), (40000, 2000)],
                         ids=["16385x16384", "8192x32769", "40000x2000"])
def test_symmetric_large_by_intersection(serac, nA, nB):
    """Prepared-path and wide pairs: symmetric = cross(A, B) and the
    transposed cross(B, A), from the library's default path."""
    p = synth.pair(nA, nB, 0.2, 4, seed=nA % 97)
    a, b = dev(p.A), dev(p.B)
    say(f"[variants] large symmetric {nA}x{nB}")
    for r in (0.8, 1.2):
        sym = serac.match_pair(a, b, r, math.inf, True, symmetric=True)
        fwd = _set(serac.match_pair(a, b, r, math.inf, True))
        rev = {(j, i) for i, j in _set(serac.match_pair(b, a, r, math.inf, True))}
        assert _set(sym) == fwd & rev, (nA, nB, r)
        s = sym.cpu().numpy()
        assert np.all(np.diff(s[:, 0]) > 0)
    # a sample of rows settled by the oracle one by one, in both directions
    rows = np.linspace(0, nA - 1, 64).astype(np.int32)
    want = oracle.match_rows(p.A, p.B, rows, 0.8)
    got = {i: j for i, j in _set(serac.match_pair(a, b, 0.8, math.inf, True, symmetric=True))}
    for i, j in want.items():
        if j < 0:
            assert i not in got
        else:
            # the row passes its own gates and the mutual check; the column
            # gate can only remove it
            assert got.get(i, j) == j


def test_cap_single_pair(serac):
    p = synth.pair(3000, 2600, 0.3, 4, seed=8)
    for cap in (1, 255, 1000, 2599, 2600, 2601, 10000):
        for sym in (False, True):
            check(serac, p.A, p.B, 0.8, math.inf, True, sym, cap, label=f"cap {cap}")
    check(serac, p.A, p.B, 1.2, 0.7, False, False, 777, label="cap, no cross-check")
    # the capacity needed is the capped row count
    a, b = dev(p.A), dev(p.B)
    out = torch.full((1000, 2), -7, dtype=torch.int32, device="cuda:0")
    cnt = torch.full((1,), -7, dtype=torch.int32, device="cuda:0")
    serac.match_pair_into(a, b, out, cnt, max_features=1000)
    n = int(cnt.item())
    want = oracle.match_pair(p.A, p.B, max_features=1000)
    assert out[:n].cpu().numpy().astype(np.uint32).tobytes() == want.tobytes()


def test_cap_noalloc(serac):
    serac.init()
    p = synth.pair(3000, 2600, 0.3, 4, seed=9)
    a, b = dev(p.A), dev(p.B)
    for cap in (300, 2600):
        out = torch.full((3000, 2), -7, dtype=torch.int32, device="cuda:0")
        cnt = torch.full((1,), -7, dtype=torch.int32, device="cuda:0")
        serac.match_pair_noalloc_into(a, b, out, cnt, max_features=cap)
        n = int(cnt.item())
        want = oracle.match_pair(p.A, p.B, max_features=cap)
        assert out[:n].cpu().numpy().astype(np.uint32).tobytes() == want.tobytes(), cap


def test_batch_variants(serac):
    """A batch of mixed sizes (both sides of 8192 rows, an empty and a
    one-row image) with symmetric gates, a cap, and both; device lists and
    the host pipeline's, every pair against the oracle."""
    rng = np.random.default_rng(21)
    sizes = [1500, 0, 9000, 1, 700, 2300, 256]
    imgs_np = [synth.desc(rng, n) for n in sizes]
    # plant shared rows between neighbours
    for k in range(len(sizes) - 1):
        m = min(sizes[k], sizes[k + 1]) // 5
        if m:
            imgs_np[k + 1][:m] = np.clip(imgs_np[k][:m].astype(np.int16)
                                         + rng.integers(-3, 4, (m, 128)), 0, 255)
    imgs = [dev(x) for x in imgs_np]
    pairs = [(a, b) for a in range(len(sizes)) for b in range(len(sizes)) if a != b]
    for sym, cap in ((True, 0), (False, 600), (True, 2000)):
        say(f"[variants] batch sym={sym} cap={cap}")
        got = serac.match_pairs(imgs, pairs, 0.8, math.inf, True, symmetric=sym,
                                max_features=cap)
        host = serac.match_pairs_host(imgs, pairs, 0.8, math.inf, True, pairs_per_stage=5,
                                      symmetric=sym, max_features=cap)
        for q, (a, b) in enumerate(pairs):
            want = oracle.match_pair(imgs_np[a], imgs_np[b], 0.8, math.inf, True,
                                     symmetric=sym, max_features=cap)
            g = got[q].cpu().numpy().astype(np.uint32)
            assert g.tobytes() == want.tobytes(), (sym, cap, a, b)
            assert host[q].tobytes() == want.tobytes(), (sym, cap, a, b, "host")


def test_batch_symmetric_equals_single_calls(serac):
    """The 48 x 8192 batch under symmetric gates: every pair equals its
    single-pair call, and a spread of pairs the oracle."""
    bt = synth.exhaustive_48x8192()
    imgs = [dev(x) for x in bt.images]
    pairs = bt.pairs.tolist()
    say("[variants] 48x8192 batch, symmetric")
    got = serac.match_pairs(imgs, pairs, 0.8, math.inf, True, symmetric=True)
    for q, (a, b) in enumerate(pairs):
        if q % 47 == 0:
            one = serac.match_pair(imgs[a], imgs[b], 0.8, math.inf, True, symmetric=True)
            assert torch.equal(got[q], one), (a, b)
    for q in (0, 1, 500, len(pairs) - 1):
        a, b = pairs[q]
        want = oracle.match_pair(bt.images[a], bt.images[b], 0.8, math.inf, True,
                                 symmetric=True)
        assert got[q].cpu().numpy().astype(np.uint32).tobytes() == want.tobytes(), (a, b)
