"""A host simulation of the sweep's reduction order, on tie-heavy scores.

The tile kernel never holds a row's scores together: each of the 32 lanes
that share a row sees one column per 32-column tile, keeps a running best
and runner-up of packed keys (S << 9 | 511 - t) over tile pairs with
max3 / med3 (the second-best update deferred to every other pair), the
lanes are merged pairwise in a tree (lower lane first in every pair), and the column groups of a row meet
only as packed 64-bit slots in the finishing kernel.  The column side
raises (S << 9 | 511 - slice) by atomic maxima and settles the lowest row
of a 16-row slice with bounds from the rows' own top-2.  The result must not
depend on the order any of this happens in (MASDA part 3, section 6: an
order-independent key) and must equal the plain definition: best, lowest
column of the best, second counted with multiplicity; lowest row of a
column's maximum.

Here the same steps run in NumPy, with the same bit layouts, over 0.5 M
rows of tie-heavy scores (many equal values, zero rows, columns past the end
of the set), group orders permuted, and are compared with the definition.
"""
import numpy as np

TILE = 32
CHUNK = 256
GROUP_MAX = 16384
SLOT_COL_MAX = (1 << 18) - 1
SLICE = 16


def definition_rows(S):
    """(best, idx, second) per row: identity (0, -1, 0), lowest column on a
    tie, second with multiplicity."""
    T, n = S.shape
    best = S.max(axis=1) if n else np.zeros(T, np.int64)
    idx = np.where(best > 0, np.argmax(S, axis=1), -1) if n else np.full(T, -1)
    if n >= 2:
        second = -np.partition(-S, 1, axis=1)[:, 1]
    else:
        second = np.zeros(T, np.int64)
    return best, idx, second


def lane_sweep(S, c0, ncols):
    """One workgroup's column group [c0, c0 + ncols) of every row: the
    per-lane running keys over tile pairs and the lane merge; returns the
    packed 64-bit slots.  Columns past the set (S is zero-padded by the
    caller) score 0, as the all-zero padding descriptor does."""
    T = S.shape[0]
    window = c0 & ~(GROUP_MAX - 1)
    b1 = np.zeros((T, TILE), np.uint64)
    b2 = np.zeros((T, TILE), np.uint64)
    tk = np.zeros((T, TILE), np.uint64)
    npairs = ncols // (2 * TILE)
    for p in range(npairs):
        keys = []
        for tt in range(2):
            col0 = c0 + (2 * p + tt) * TILE
            t = (col0 - window) // TILE
            s = S[:, col0:col0 + TILE].astype(np.uint64)
            keys.append((s << np.uint64(9)) | np.uint64(511 - t))
        k0, k1 = keys
        lo, hi = np.minimum(k0, k1), np.maximum(k0, k1)
        md = np.maximum(lo, np.minimum(hi, b1))      # med3(b1, k0, k1)
        b1 = np.maximum(b1, hi)                      # max3(b1, k0, k1)
        if p % 2 == 1:                               # odd pair: close the fold
            b2 = np.maximum(np.maximum(b2, tk), md)
        else:
            tk = md
    assert npairs % 2 == 0                            # a chunk is four pairs
    # lane merge: within each half (source lanes 0..15, 16..31) a pairwise
    # tree, the lower lane first in every pair; then across the halves
    K1 = np.zeros((T, 2), np.uint64)
    K2 = np.zeros((T, 2), np.uint64)
    L = np.zeros((T, 2), np.int64)
    for h in range(2):
        t1 = [b1[:, 16 * h + k] for k in range(16)]
        t2 = [b2[:, 16 * h + k] for k in range(16)]
        tl = [np.full(T, k, np.int64) for k in range(16)]
        s = 1
        while s < 16:
            for k in range(0, 16, 2 * s):
                a1, c1 = t1[k], t1[k + s]
                tl[k] = np.where(c1 > a1, tl[k + s], tl[k])
                t2[k] = np.maximum(np.maximum(np.minimum(a1, c1), t2[k]), t2[k + s])
                t1[k] = np.maximum(a1, c1)
            s *= 2
        K1[:, h], K2[:, h], L[:, h] = t1[0], t2[0], 16 * h + tl[0]
    # half 0 keeps its own on a key tie (it holds the lower lanes)
    o1, o2, oL = K1[:, 1], K2[:, 1], L[:, 1]
    A1, A2, AL = K1[:, 0], K2[:, 0], L[:, 0]
    L1 = np.where(o1 > A1, oL, AL)
    K2f = np.maximum(np.maximum(np.minimum(A1, o1), A2), o2)
    K1f = np.maximum(A1, o1)
    S1 = K1f >> np.uint64(9)
    S2 = K2f >> np.uint64(9)
    col = window + TILE * (511 - (K1f & np.uint64(511)).astype(np.int64)) + L1
    slot = (S1 << np.uint64(41)) | (np.uint64(SLOT_COL_MAX) - col.astype(np.uint64)) \
        << np.uint64(23) | S2
    return np.where(S1 == 0, np.uint64(0), slot)


def row_result(slots):
    """The finishing kernel's merge of a row's slots, in the order given."""
    best = np.zeros(slots.shape[0], np.uint64)
    sec = np.zeros(slots.shape[0], np.uint64)
    loser = np.zeros(slots.shape[0], np.uint64)
    for v in slots.T:
        lo = np.minimum(best, v)
        loser = np.maximum(loser, lo >> np.uint64(41))
        best = np.maximum(best, v)
        sec = np.maximum(sec, v & np.uint64(0x7FFFFF))
    S1 = (best >> np.uint64(41)).astype(np.int64)
    I1 = np.where(S1 > 0, SLOT_COL_MAX - ((best >> np.uint64(23)) & np.uint64(SLOT_COL_MAX))
                  .astype(np.int64), -1)
    return S1, I1, np.maximum(sec, loser).astype(np.int64)


def tie_heavy_scores(rng, T, n):
    """Scores from a handful of values (many exact ties, whole zero rows),
    a few large ones near the 23-bit limit."""
    kind = rng.integers(0, 4, size=(T, 1))
    small = rng.integers(0, 4, size=(T, n))
    mid = rng.choice(np.array([0, 7, 7, 1000, 1000, 1001]), size=(T, n))
    big = rng.integers((1 << 23) - 40, (1 << 23) - 1, size=(T, n))
    S = np.where(kind == 0, small, np.where(kind == 1, mid, np.where(kind == 2, big, 0)))
    zero_rows = rng.random(T) < 0.03
    S[zero_rows] = 0
    return S.astype(np.int64)


def run_rows(rng, T, n, gch, shuffle_groups):
    S = tie_heavy_scores(rng, T, n)
    width = gch * CHUNK
    ngroups = -(-n // width)
    padded = np.zeros((T, ngroups * width), np.int64)
    padded[:, :n] = S
    slots = np.stack([lane_sweep(padded, g * width, width) for g in range(ngroups)], axis=1)
    if shuffle_groups:
        slots = slots[:, rng.permutation(ngroups)]
    got = row_result(slots)
    want = definition_rows(S)
    for a, b, what in zip(got, want, ("best", "idx", "second")):
        assert np.array_equal(a, b), (n, gch, what, np.flatnonzero(a != b)[:5])
    return T


def test_row_reduction_half_a_million_rows():
    rng = np.random.default_rng(2024)
    trials = 0
    # (rows, columns, chunks per column group): ragged tails, one and many
    # groups, groups in the 16384-column window's upper half
    for T, n, gch in ((160000, 7, 1), (150000, 33, 1), (100000, 256, 1), (60000, 300, 1),
                      (20000, 777, 2), (8000, 1500, 4), (4000, 2049, 1),
                      (2000, 4100, 8), (1200, 9000, 2), (600, 17000, 64)):
        trials += run_rows(rng, T, n, gch, shuffle_groups=True)
    assert trials >= 500000


def test_single_column_and_all_zero():
    rng = np.random.default_rng(1)
    run_rows(rng, 1000, 1, 1, False)
    S = np.zeros((5, 300), np.int64)
    padded = np.zeros((5, 512), np.int64)
    padded[:, :300] = S
    s1, i1, s2 = row_result(np.stack([lane_sweep(padded, 0, 256),
                                      lane_sweep(padded, 256, 256)], axis=1))
    assert (s1 == 0).all() and (i1 == -1).all() and (s2 == 0).all()


# ------------------------------------------------------------- column side
def column_side(S, row_top2):
    """The cross-check as the sweep and the finishing kernel take it, for a
    whole matrix: column bests as the maximum of (S << 9 | 511 - slice) over
    rows (what the atomic maxima leave, whatever their order), then for each
    row its best column's (C1, slice) and the slice test with the row
    bounds; the exact product only where the bounds leave it open."""
    nA, nB = S.shape
    best, idx, second = row_top2
    slices = np.arange(nA) // SLICE
    packed = (S.astype(np.int64) << 9) | (511 - slices)[:, None]
    cb = packed.max(axis=0)
    C1all, slall = cb >> 9, 511 - (cb & 511)
    acc = np.zeros(nA, bool)
    exact_calls = 0
    for i in range(nA):
        j = idx[i]
        if j < 0:
            continue
        C1, sl = C1all[j], slall[j]
        ok = C1 == best[i] and sl == i // SLICE
        if not ok:
            continue
        tie = False
        for i2 in range(sl * SLICE, i):
            if idx[i2] == j:
                tie |= best[i2] == C1
            elif best[i2] >= C1 and second[i2] >= C1:
                exact_calls += 1
                tie |= S[i2, j] == C1
        acc[i] = not tie
    return acc, exact_calls


def test_cross_check_slice_ties():
    """Mutual best by the slice logic == lowest row of the column maximum."""
    rng = np.random.default_rng(77)
    total = exact = 0
    for trial in range(400):
        nA = int(rng.integers(1, 80))
        nB = int(rng.integers(1, 40))
        S = tie_heavy_scores(rng, nA, nB)
        if trial % 3 == 0:                       # duplicated rows: column ties
            S[1::2] = S[0::2][: S[1::2].shape[0]]
        rt = definition_rows(S)
        acc, e = column_side(S, rt)
        exact += e
        cmax = S.max(axis=0)
        lowest = np.argmax(S == cmax[None, :], axis=0)
        want = np.array([rt[1][i] >= 0 and lowest[rt[1][i]] == i for i in range(nA)])
        assert np.array_equal(acc, want), trial
        total += nA
    assert total > 10000 and exact > 0
