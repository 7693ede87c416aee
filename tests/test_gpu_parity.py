"""The HIP path against the CPU oracle, through the C ABI.

Match lists must be byte-identical (uint32 pairs, ascending row) and the
top-2 export must equal the oracle's row top-2 and column best exactly:
every score is an integer and the gates are one fixed double expression.
Sizes span several 256-row blocks and 512-column chunks with ragged tails;
the full-size workloads are checked in full where the oracle finishes in
seconds (8192 x 8192) and on sampled rows and columns otherwise.
"""
import hashlib
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


def check_pair(serac, A, B, max_ratio=0.8, max_distance=math.inf, cross_check=True,
               top2=True, label=""):
    say(f"[parity] {label} nA={len(A)} nB={len(B)} ratio={max_ratio} "
        f"dist={max_distance} cross={cross_check}")
    a, b = dev(A), dev(B)
    got = serac.match_pair(a, b, max_ratio, max_distance, cross_check)
    got = got.cpu().numpy().astype(np.uint32)
    want = oracle.match_pair(A, B, max_ratio, max_distance, cross_check)
    assert got.shape == want.shape, (label, got.shape, want.shape)
    assert got.tobytes() == want.tobytes(), label
    if top2:
        row, col = serac.top2(a, b)
        orow, ocol = oracle.top2(A, B)
        assert_rows_equal(row.cpu().numpy(), orow, label + " row_top2")
        assert_rows_equal(col.cpu().numpy(), ocol, label + " col_best")
    return got


def assert_rows_equal(got, want, label):
    """Exact equality with the first differing rows named on failure."""
    assert got.shape == want.shape, (label, got.shape, want.shape)
    bad = np.flatnonzero((got != want).any(axis=1))
    assert bad.size == 0, (f"{label}: {bad.size} rows differ, first "
                           f"{[(int(i), got[i].tolist(), want[i].tolist()) for i in bad[:6]]}")


SMALL = [(1, 1), (1, 2), (2, 1), (3, 17), (17, 3), (40, 40), (255, 511), (256, 512),
         (257, 513), (300, 1100), (1029, 777), (513, 1537)]


@pytest.mark.parametrize("nA,nB", SMALL, ids=[f"{a}x{b}" for a, b in SMALL])
def test_tie_heavy_small(serac, nA, nB):
    rng = np.random.default_rng(nA * 7919 + nB)
    A = tie_heavy(rng, nA)
    B = tie_heavy(rng, nB)
    for r, cc in ((0.8, True), (1.5, True), (0.8, False)):
        check_pair(serac, A, B, r, math.inf, cc, top2=(r == 0.8 and cc),
                   label=f"tie-heavy {nA}x{nB}")


@pytest.mark.parametrize("nA,nB", [(1000, 1200), (700, 2100), (2048, 96), (96, 2048),
                                   (4099, 1031)])
def test_planted_pairs(serac, nA, nB):
    p = synth.pair(nA, nB, 0.3, 3, seed=nA + nB)
    got = check_pair(serac, p.A, p.B, label=f"planted {nA}x{nB}")
    assert len(got) > 0


def _random_case(k):
    """Case k of the seeded sweep: a shape near a tile boundary or arbitrary,
    one of four generators, and one setting of the gates."""
    rng = np.random.default_rng(10_000 + k)

    def size(hi):
        if rng.random() < 0.5:                   # next to a 32-, 256- or 512-multiple
            m = int(rng.choice([32, 256, 512]))
            return int(max(1, m * rng.integers(1, hi // m + 1) + rng.integers(-1, 2)))
        return int(rng.integers(1, hi + 1))
    nA, nB = size(2600), size(4700)
    kind = ("planted", "tie", "random", "coarse")[k % 4]
    if kind == "planted":
        p = synth.pair(nA, nB, 0.3, 3, seed=k)
        A, B = p.A, p.B
    elif kind == "tie":
        A, B = tie_heavy(rng, nA), tie_heavy(rng, nB)
    elif kind == "random":
        A, B = synth.desc(rng, nA), synth.desc(rng, nB)
    else:                                        # bytes 0 or 45: scores are multiples of 2025
        A = (rng.integers(0, 2, (nA, 128)) * 45).astype(np.uint8)
        B = (rng.integers(0, 2, (nB, 128)) * 45).astype(np.uint8)
    if kind in ("tie", "coarse"):                # lenient gates, so that tied bests can pass
        ratio = float(rng.choice([1.0, 1.3]))
        dist = math.inf if kind == "tie" else float(rng.choice([math.inf, 1.2]))
    else:
        ratio = float(rng.choice([0.6, 0.8, 1.0, 1.3]))
        dist = float(rng.choice([math.inf, 0.3, 0.7]))
    cross = bool(rng.random() < 0.7)
    return kind, A, B, ratio, dist, cross


@pytest.mark.parametrize("k", range(40))
def test_random_sweep(serac, k):
    kind, A, B, ratio, dist, cross = _random_case(k)
    check_pair(serac, A, B, ratio, dist, cross, top2=(k % 3 == 0),
               label=f"sweep {k} {kind}")


def test_workload_pair_1000x1200(serac):
    p = synth.workload("pair_1000x1200")
    got = check_pair(serac, p.A, p.B, **p.params(), label=p.name)
    assert {tuple(x) for x in got.astype(np.int64).tolist()} == \
        {tuple(x) for x in p.truth.tolist()}


def test_workload_pair_8192x8192(serac):
    p = synth.workload("pair_8192x8192")
    check_pair(serac, p.A, p.B, **p.params(), label=p.name)


@pytest.mark.parametrize("name", ["edge_8192x8192_ties", "edge_8192x8192_ties_no255",
                                  "edge_8192x96_skinny", "edge_8192x96_skinny_no255"])
def test_workload_edges(serac, name):
    p = synth.workload(name)
    check_pair(serac, p.A, p.B, **p.params(), label=name)
    # the same pair through the other gates
    check_pair(serac, p.A, p.B, 1.25, 0.7, True, top2=False, label=name + " r1.25 d0.7")
    check_pair(serac, p.A, p.B, 0.8, math.inf, False, top2=False, label=name + " nocc")


def test_empty_sides(serac):
    rng = np.random.default_rng(5)
    A = synth.desc(rng, 10)
    E = np.zeros((0, 128), np.uint8)
    for X, Y in ((A, E), (E, A), (E, E)):
        a, b = dev(X), dev(Y)
        assert serac.match_pair(a, b).shape[0] == 0
        row, col = serac.top2(a, b)
        assert row.cpu().tolist() == [[0, -1, 0]] * len(X)
        assert col.cpu().tolist() == [[0, -1]] * len(Y)


def test_zero_and_saturated_rows(serac):
    A = np.zeros((300, 128), np.uint8)
    B = np.zeros((600, 128), np.uint8)
    A[17] = 255
    A[200] = 255          # a duplicate: the column best must be row 17
    B[599] = 255
    B[3] = 1
    check_pair(serac, A, B, label="zeros/255")


def test_slice_column_ties(serac):
    """Cross-check ties inside one 16-row slice: a lower row of the slice on
    the same column with the same best score (duplicate rows), and a lower
    row whose best is another column but whose second reaches the column
    maximum, once tying on the column (the match is refused) and once just
    below it (the match stands)."""
    rng = np.random.default_rng(21)
    A = synth.desc(rng, 300) // 4        # low scores everywhere else
    B = synth.desc(rng, 200) // 4
    def blk(k, v=255):
        x = np.zeros(128, np.uint8)
        x[4 * k:4 * k + 4] = v
        return x
    # slice 0: rows 2 and 9 both see column 5 (k = 1) as their only good column
    B[5] = blk(1)
    A[2] = blk(1)
    A[9] = blk(1)
    # slice 1: row 17 ties columns 7 and 8 (k = 2, 3); row 20 sees column 8
    B[7] = blk(2)
    B[8] = blk(3)
    A[17] = blk(2) | blk(3)
    A[20] = blk(3)
    # slice 2: row 33 ties columns 10 and 12 (k = 4, twice) and scores just
    # below the maximum on column 11 (k = 5); row 40 sees column 11
    B[10] = blk(4)
    B[12] = blk(4)
    B[11] = blk(5)
    A[33] = blk(4) | blk(5, 254)
    A[40] = blk(5)
    got = check_pair(serac, A, B, label="slice column ties")
    pairs = {tuple(x) for x in got.astype(np.int64).tolist()}
    assert (2, 5) in pairs and (9, 5) not in pairs
    assert (20, 8) not in pairs
    assert (40, 11) in pairs


def test_determinism_and_stream(serac):
    """20 runs on a side stream, each into an output poisoned with 0xFF
    bytes and a count of -7: the same SHA-256 every time, the oracle's list,
    and nothing written past the count."""
    p = synth.workload("edge_8192x8192_ties_no255")
    a, b = dev(p.A), dev(p.B)
    s = torch.cuda.Stream()
    digests = set()
    first = None
    for k in range(20):
        out = torch.full((p.A.shape[0], 2), -1, dtype=torch.int32, device="cuda:0")
        cnt = torch.full((1,), -7, dtype=torch.int32, device="cuda:0")
        with torch.cuda.stream(s):
            serac.match_pair_into(a, b, out, cnt)
        s.synchronize()
        n = int(cnt.item())
        full = out.cpu().numpy()
        assert (full[n:] == -1).all(), k
        digests.add(hashlib.sha256(full[:n].tobytes()).hexdigest())
        first = full[:n].tobytes() if first is None else first
    assert len(digests) == 1
    want = oracle.match_pair(p.A, p.B, 0.8, math.inf, True)
    assert first == want.tobytes()


def test_pipelined_calls_identical(serac):
    """30 calls in flight on one stream with no synchronisation between
    them, alternating three pairs of different shapes and paths (fused
    32-bit, fused 64-bit column bests, prepared), each into its own output:
    every list is the oracle's.  Consecutive calls share the workspace's
    accumulator regions (each call clears what the one before left), so a
    race between calls would show here (the pages' 30 pipelined frames)."""
    cases = [synth.workload("edge_8192x8192_ties_no255"),
             synth.pair(9000, 5000, 0.2, 4, seed=6),         # > 8192 rows: 64-bit column bests
             synth.pair(16385, 16384, 0.1, 4, seed=7)]       # > 2^28 products: prepared sets
    dv = [(dev(c.A), dev(c.B)) for c in cases]
    want = [oracle.match_pair(c.A, c.B, 0.8, math.inf, True).tobytes() for c in cases]
    outs = []
    torch.cuda.synchronize()
    for k in range(30):
        a, b = dv[k % 3]
        out = torch.full((a.shape[0], 2), -1, dtype=torch.int32, device="cuda:0")
        cnt = torch.full((1,), -7, dtype=torch.int32, device="cuda:0")
        serac.match_pair_into(a, b, out, cnt)
        outs.append((out, cnt))
    torch.cuda.synchronize()
    for k, (out, cnt) in enumerate(outs):
        got = out[: int(cnt.item())].cpu().numpy().tobytes()
        assert got == want[k % 3], k


def test_workload_pair_32768_sampled(serac):
    p = synth.workload("pair_32768x32768")
    a, b = dev(p.A), dev(p.B)
    say("[parity] pair_32768x32768 GPU")
    got = serac.match_pair(a, b, **p.params()).cpu().numpy().astype(np.int64)
    row, col = serac.top2(a, b)
    row, col = row.cpu().numpy(), col.cpu().numpy()
    rng = np.random.default_rng(11)
    sample = np.unique(np.concatenate([rng.choice(len(p.A), 192, replace=False),
                                       p.truth[:64, 0], [0, len(p.A) - 1]])).astype(np.int32)
    say(f"[parity] pair_32768x32768 oracle on {len(sample)} sampled rows")
    dec = oracle.match_rows(p.A, p.B, sample, **p.params())
    gmap = {int(x[0]): int(x[1]) for x in got}
    for i in sample.tolist():
        assert gmap.get(i, -1) == dec[i], i
    assert np.array_equal(row[sample], oracle.rows(p.A, p.B, sample))
    csample = np.unique(np.concatenate([rng.choice(len(p.B), 192, replace=False),
                                        p.truth[:64, 1], [len(p.B) - 1]])).astype(np.int32)
    assert np.array_equal(col[csample], oracle.cols(p.A, p.B, csample))
    # properties at full size: sorted, one-to-one, mutual
    assert np.all(np.diff(got[:, 0]) > 0)
    assert len(np.unique(got[:, 1])) == len(got)
    assert np.all(row[got[:, 0], 1] == got[:, 1]) and np.all(col[got[:, 1], 1] == got[:, 0])
    assert {tuple(x) for x in p.truth.tolist()} <= {tuple(x) for x in got.tolist()}


def test_max_size_sampled(serac):
    """The largest accepted set (SERAC_MAX_DESCRIPTORS = 262144 rows of A)
    against 262143 rows of B (16 column groups of 16384 columns, a ragged
    last chunk, 1024 finishing workgroups): sampled rows and columns against
    the oracle, whole-list properties at full size."""
    say("[parity] max size: generating 262144 x 262143")
    p = synth.pair(262144, 262143, 0.02, 3, seed=262)
    a, b = dev(p.A), dev(p.B)
    say("[parity] max size: GPU match and top-2 export")
    got = serac.match_pair(a, b, 0.8, math.inf, True).cpu().numpy().astype(np.int64)
    row, col = serac.top2(a, b)
    row, col = row.cpu().numpy(), col.cpu().numpy()
    rng = np.random.default_rng(12)
    sample = np.unique(np.concatenate([rng.choice(len(p.A), 96, replace=False),
                                       p.truth[:32, 0], [0, len(p.A) - 1]])).astype(np.int32)
    say(f"[parity] max size: oracle on {len(sample)} sampled rows")
    dec = oracle.match_rows(p.A, p.B, sample, 0.8, math.inf, True)
    gmap = {int(x[0]): int(x[1]) for x in got}
    for i in sample.tolist():
        assert gmap.get(i, -1) == dec[i], i
    assert np.array_equal(row[sample], oracle.rows(p.A, p.B, sample))
    csample = np.unique(np.concatenate([rng.choice(len(p.B), 96, replace=False),
                                        p.truth[:32, 1], [len(p.B) - 1]])).astype(np.int32)
    assert np.array_equal(col[csample], oracle.cols(p.A, p.B, csample))
    assert np.all(np.diff(got[:, 0]) > 0)
    assert len(np.unique(got[:, 1])) == len(got)
    assert np.all(row[got[:, 0], 1] == got[:, 1]) and np.all(col[got[:, 1], 1] == got[:, 0])
    assert {tuple(x) for x in p.truth.tolist()} <= {tuple(x) for x in got.tolist()}


def test_batch_48x8192(serac):
    bt = synth.exhaustive_48x8192()
    imgs = [dev(x) for x in bt.images]
    say(f"[parity] batch {len(bt.pairs)} pairs")
    res = serac.match_pairs(imgs, bt.pairs.tolist(), **bt.params())
    assert len(res) == len(bt.pairs)
    # the same lists delivered to host memory by the host pipeline
    host = serac.match_pairs_host(imgs, bt.pairs.tolist(), **bt.params())
    for k in range(len(bt.pairs)):
        assert host[k].tobytes() == res[k].cpu().numpy().astype(np.uint32).tobytes(), k
    # every pair equals the single-pair call on it
    for k, (ia, ib) in enumerate(bt.pairs.tolist()):
        one = serac.match_pair(imgs[ia], imgs[ib], **bt.params())
        assert torch.equal(one, res[k]), (ia, ib)
    # the oracle on a few pairs in full
    for ia, ib in ((0, 1), (0, 2), (20, 47)):
        k = int(np.flatnonzero((bt.pairs[:, 0] == ia) & (bt.pairs[:, 1] == ib))[0])
        say(f"[parity] batch pair ({ia},{ib}) vs oracle")
        want = oracle.match_pair(bt.images[ia], bt.images[ib], **bt.params())
        assert res[k].cpu().numpy().astype(np.uint32).tobytes() == want.tobytes()
        if (ia, ib) in bt.truth:
            t = {tuple(x) for x in bt.truth[(ia, ib)].tolist()}
            assert t <= {tuple(x) for x in want.astype(np.int64).tolist()}


def test_pairs_host_mixed(serac):
    """serac_match_pairs_host: stages of 3 pairs (both halves of its double
    buffer reused several times, the last stage partial), of 64 (one stage)
    and the default, on images of mixed sizes including an empty one and a
    one-row one; every list equals match_pairs', a few the oracle's."""
    rng = np.random.default_rng(17)
    sizes = (700, 0, 1300, 257, 2048, 1)
    imgs_np = [synth.desc(rng, n) for n in sizes]
    for k in (2, 3, 4):
        imgs_np[k][:30] = synth.noisy(rng, imgs_np[0][30 * k:30 * k + 30], 3)
    imgs = [dev(x) for x in imgs_np]
    pairs = [(a, b) for a in range(len(sizes)) for b in range(len(sizes)) if a != b]
    ref = [x.cpu().numpy().astype(np.uint32) for x in
           serac.match_pairs(imgs, pairs, 0.8, 0.7, True)]
    assert sum(len(x) for x in ref) > 0
    for per in (3, 64, 0):
        say(f"[parity] host pipeline, {len(pairs)} pairs, stages of {per}")
        res = serac.match_pairs_host(imgs, pairs, 0.8, 0.7, True, pairs_per_stage=per)
        assert len(res) == len(pairs)
        for k in range(len(pairs)):
            assert res[k].dtype == np.uint32 and res[k].shape[1:] == (2,)
            assert res[k].tobytes() == ref[k].tobytes(), (per, pairs[k])
    for a, b in ((0, 2), (2, 0), (3, 4), (0, 1), (5, 0)):
        want = oracle.match_pair(imgs_np[a], imgs_np[b], 0.8, 0.7, True)
        assert res[pairs.index((a, b))].tobytes() == want.tobytes(), (a, b)


def test_batch_mixed_sizes(serac):
    """A batch whose images straddle 8192 rows: pairs whose first image has
    more than 8192 rows need 64-bit column bests, so the whole batch uses
    them; every pair against the oracle, cross-check on and off."""
    rng = np.random.default_rng(91)
    sizes = (9000, 300, 1200, 8192)
    imgs_np = [synth.desc(rng, n) for n in sizes]
    # plant shared rows so that every pair matches some
    for k in range(1, len(sizes)):
        imgs_np[k][:40] = imgs_np[0][:40]
        imgs_np[k][40:60] = imgs_np[0][k * 50:k * 50 + 20]
    imgs = [dev(x) for x in imgs_np]
    pairs = [(a, b) for a in range(len(sizes)) for b in range(len(sizes)) if a != b]
    for cross in (True, False):
        say(f"[parity] mixed-size batch, cross-check {cross}")
        res = serac.match_pairs(imgs, pairs, 0.8, math.inf, cross)
        for k, (a, b) in enumerate(pairs):
            want = oracle.match_pair(imgs_np[a], imgs_np[b], 0.8, math.inf, cross)
            assert res[k].cpu().numpy().astype(np.uint32).tobytes() == want.tobytes(), (a, b)
    # without the large image the batch keeps 32-bit column bests
    small = [1, 2, 3]
    pairs2 = [(a, b) for a in small for b in small if a != b]
    res = serac.match_pairs(imgs, pairs2, 0.8, math.inf, True)
    for k, (a, b) in enumerate(pairs2):
        want = oracle.match_pair(imgs_np[a], imgs_np[b], 0.8, math.inf, True)
        assert res[k].cpu().numpy().astype(np.uint32).tobytes() == want.tobytes(), (a, b)


# A single pair is swept straight from the raw descriptors up to 2^28
# products and through the preparation kernel above; both sides of the
# switch, with ragged tails.
FUSED_LIMIT = 1 << 28


@pytest.mark.parametrize("nA,nB", [(16384, 16384), (16385, 16384), (8192, 32769)],
                         ids=["16384x16384", "16385x16384", "8192x32769"])
def test_fused_switch(serac, nA, nB):
    path = "fused" if nA * nB <= FUSED_LIMIT else "prepared"
    p = synth.pair(nA, nB, 0.2, 4, seed=nA ^ nB)
    got = check_pair(serac, p.A, p.B, 0.8, 0.7, True, top2=(nA <= 8192),
                     label=f"switch {nA}x{nB} ({path})")
    assert len(got) > 0


@pytest.mark.parametrize("nA,nB", [(10400, 10400), (12000, 12000), (4096, 32769)],
                         ids=["10400sq", "12000sq", "4096x32769"])
def test_column_group_plans(serac, nA, nB):
    """Pairs whose column-group size comes from the sweep-round estimate:
    10400^2 (fused, 8-chunk groups and a ragged 1-chunk group in one
    round), 12000^2 (prepared, 4-chunk groups over three rounds and a
    ragged 3-chunk group), 4096 x 32769 (prepared, 8-chunk groups and a
    ragged group in a second round)."""
    p = synth.pair(nA, nB, 0.2, 4, seed=nA + 7 * nB)
    got = check_pair(serac, p.A, p.B, 0.8, 0.7, True, top2=False, label=f"plan {nA}x{nB}")
    assert len(got) > 0


def test_wide_column_groups(serac):
    """A tall pair gets 64-chunk (16384-column) column groups: column maxima
    leave the 8-chunk LDS ring during the sweep, tile tags use all 9 bits,
    and the last group is a single ragged chunk."""
    p = synth.pair(65536, 16384 + 100, 0.05, 3, seed=65)
    check_pair(serac, p.A, p.B, 0.8, 0.7, True, top2=True, label="wide groups 65536x16484")


def test_mixed_calls_one_stream(serac):
    """Fused and prepared sweeps, a batch and a top-2 export in turn on one
    stream share one workspace; every call starts from clean accumulators."""
    rng = np.random.default_rng(77)
    small = synth.pair(700, 900, 0.3, 3, seed=5)
    big = synth.pair(4096, 32769, 0.2, 4, seed=6)
    imgs_np = [synth.desc(rng, n) for n in (300, 520, 800)]
    imgs = [dev(x) for x in imgs_np]
    pairs = [(0, 1), (1, 2), (2, 0)]
    want_small = oracle.match_pair(small.A, small.B, 0.8, math.inf, True)
    want_big = oracle.match_pair(big.A, big.B, 0.8, math.inf, True)
    want_batch = [oracle.match_pair(imgs_np[a], imgs_np[b], 0.8, math.inf, True)
                  for a, b in pairs]
    orow, ocol = oracle.top2(small.A, small.B)
    sa, sb, ba, bb = dev(small.A), dev(small.B), dev(big.A), dev(big.B)
    for rep in range(2):
        say(f"[mixed] round {rep}")
        got = serac.match_pair(sa, sb).cpu().numpy().astype(np.uint32)
        assert got.tobytes() == want_small.tobytes(), ("fused", rep)
        got = serac.match_pair(ba, bb).cpu().numpy().astype(np.uint32)
        assert got.tobytes() == want_big.tobytes(), ("prepared", rep)
        res = serac.match_pairs(imgs, pairs)
        for k in range(len(pairs)):
            assert res[k].cpu().numpy().astype(np.uint32).tobytes() == want_batch[k].tobytes(), \
                ("batch", rep, k)
        row, col = serac.top2(sa, sb)
        assert_rows_equal(row.cpu().numpy(), orow, f"top2 rows {rep}")
        assert_rows_equal(col.cpu().numpy(), ocol, f"top2 cols {rep}")
        got = serac.match_pair(sa, sb, 0.8, math.inf, False).cpu().numpy().astype(np.uint32)
        assert got.tobytes() == oracle.match_pair(small.A, small.B, 0.8, math.inf,
                                                  False).tobytes(), ("no cross-check", rep)


def test_two_streams(serac):
    """Calls on two streams interleave (one workspace per stream); from two
    host threads as well."""
    import threading
    p1 = synth.pair(1500, 1300, 0.3, 3, seed=31)
    p2 = synth.pair(900, 2500, 0.3, 3, seed=32)
    want = [oracle.match_pair(p.A, p.B, 0.8, math.inf, True) for p in (p1, p2)]
    dv = [(dev(p.A), dev(p.B)) for p in (p1, p2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[None] * 4 for _ in range(2)]

    def run(k, reps):
        with torch.cuda.stream(streams[k]):
            a, b = dv[k]
            for r in range(reps):
                out = torch.full((a.shape[0], 2), -1, dtype=torch.int32, device="cuda:0")
                cnt = torch.full((1,), -7, dtype=torch.int32, device="cuda:0")
                serac.match_pair_into(a, b, out, cnt)
                outs[k][r] = (out, cnt)
    for r in range(4):                       # interleaved on one host thread
        run(0, 1) if r % 2 == 0 else run(1, 1)
    torch.cuda.synchronize()
    th = [threading.Thread(target=run, args=(k, 4)) for k in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    torch.cuda.synchronize()
    for k in range(2):
        for out, cnt in outs[k]:
            n = int(cnt.item())
            assert out[:n].cpu().numpy().astype(np.uint32).tobytes() == want[k].tobytes(), k


def test_threads_one_stream(serac):
    """Two host threads calling on the same stream share its workspace; the
    library serializes their enqueues, also while one of them grows it (a
    fused pair and a larger prepared pair in turn)."""
    import threading
    p1 = synth.pair(1500, 1300, 0.3, 3, seed=41)
    p2 = synth.pair(2600, 104000, 0.2, 3, seed=42)      # above 2^28 products: prepared
    want = [oracle.match_pair(p.A, p.B, 0.8, math.inf, True) for p in (p1, p2)]
    dv = [(dev(p.A), dev(p.B)) for p in (p1, p2)]
    stream = torch.cuda.Stream()
    reps = 6
    outs = [[None] * reps for _ in range(2)]

    def run(k):
        with torch.cuda.stream(stream):
            a, b = dv[k]
            for r in range(reps):
                out = torch.full((a.shape[0], 2), -1, dtype=torch.int32, device="cuda:0")
                cnt = torch.full((1,), -7, dtype=torch.int32, device="cuda:0")
                serac.match_pair_into(a, b, out, cnt)
                outs[k][r] = (out, cnt)
    say("[threads] two host threads, one stream")
    th = [threading.Thread(target=run, args=(k,)) for k in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    torch.cuda.synchronize()
    for k in range(2):
        for r, (out, cnt) in enumerate(outs[k]):
            n = int(cnt.item())
            assert out[:n].cpu().numpy().astype(np.uint32).tobytes() == want[k].tobytes(), (k, r)


def test_lookback_failure_reported():
    """The finishing kernel's bounded look-back: with the host forcing it to
    give up at once (SERAC_LOOKBACK_SPIN_LIMIT=-1, read at the first call),
    the count is -1 and the binding raises, also through the host pipeline;
    every kernel still exits normally.  Its own process, so the setting
    stays out of the others."""
    import os
    import subprocess
    code = (
        "import sys, torch, numpy as np\n"
        "sys.path.insert(0, %r)\n"
        "import sift_descriptor_nearest_amd as serac\n"
        "from sift_descriptor_nearest_amd import synth\n"
        "p = synth.pair(700, 500, 0.3, 3, seed=3)\n"
        "a = torch.from_numpy(p.A).cuda(); b = torch.from_numpy(p.B).cuda()\n"
        "out = torch.empty((700, 2), dtype=torch.int32, device='cuda')\n"
        "cnt = torch.full((1,), 7, dtype=torch.int32, device='cuda')\n"
        "serac.match_pair_into(a, b, out, cnt)\n"
        "print('count', int(cnt.item()), flush=True)\n"
        "try:\n"
        "    serac.match_pair(a, b)\n"
        "    print('no error', flush=True)\n"
        "except serac.SeracError as e:\n"
        "    print('raised', e, flush=True)\n"
        "try:\n"
        "    serac.match_pairs_host([a, b], [(0, 1), (1, 0)], pairs_per_stage=1)\n"
        "    print('host: no error', flush=True)\n"
        "except serac.SeracError as e:\n"
        "    print('host: raised', e, flush=True)\n"
    ) % (str(__import__('pathlib').Path(__file__).resolve().parents[1]),)
    env = dict(os.environ, SERAC_LOOKBACK_SPIN_LIMIT="-1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=180)
    say(r.stdout.strip())
    assert r.returncode == 0, r.stderr[-2000:]
    assert "count -1" in r.stdout and "raised" in r.stdout, r.stdout
    assert "host: raised" in r.stdout, r.stdout


def test_binding_stream_is_torch_current(serac):
    """The binding's raw stream handle is torch's current stream, on the
    default stream and inside a side-stream context."""
    from sift_descriptor_nearest_amd import _stream
    d = torch.device("cuda:0")
    assert _stream(d) == torch.cuda.current_stream(d).cuda_stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert _stream(d) == s.cuda_stream == torch.cuda.current_stream(d).cuda_stream
    assert _stream(torch.device("cuda")) == torch.cuda.current_stream().cuda_stream


def test_profiled_launches_exact(serac):
    """Tile launches timed with dispatch-attached events give the same
    results, and the timing is returned for each of them."""
    p = synth.workload("pair_1000x1200")
    serac.profile_start(8)
    check_pair(serac, p.A, p.B, **p.params(), label="profiled")
    ms, n, per, name = serac.profile_stop()
    assert n == 2 and 0.0 < ms < 1000.0      # one match_pair and one top2 launch
    assert len(per) == 2 and abs(sum(per) - ms) < 1e-3 * max(ms, 1.0)
    assert name == "serac_tiles_fused<true, true>"
    serac.profile_start(8, 3)                # every third launch: the 1st and the 4th
    for _ in range(5):
        serac.match_pair(dev(p.A), dev(p.B), **p.params())
    ms, n, per, name = serac.profile_stop()
    assert n == 2 and 0.0 < ms < 1000.0 and len(per) == 2
    # a large pair runs the prepared sweep
    big = synth.pair(16385, 16384, 0.2, 4, seed=3)
    serac.profile_start(4)
    serac.match_pair(dev(big.A), dev(big.B), 0.8, math.inf, False)
    ms, n, per, name = serac.profile_stop()
    assert n == 1 and name == "serac_tiles_one<false, false>"
