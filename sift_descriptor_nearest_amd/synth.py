"""Seeded synthetic SIFT-like descriptor sets (input generation only).

This module builds the inputs that both the HIP library and the CPU oracle
consume.  It holds none of the matcher's arithmetic: no dot products, no
top-2, no gates.  It only draws descriptors and plants known
correspondences so that the match lists have a known ground truth.

Descriptor model.  The SERAC README (section "What changed") describes 128
unsigned 8-bit components per SIFT descriptor.  Real extraction produces
gradient-orientation histograms (Kumar, Muknahallipatna & McInroy, "An
Approach to Parallelization of SIFT Algorithm on GPUs", section on
orientation assignment and the descriptor).  As a stand-in we draw
|N(0,1)|^128, scale each vector to L2 norm 512, round half to even and clamp
to [0, 255].  The surveys the README matches (a 589-image UAV survey, a
40-image south-building subset) are not available, so these arrays stand in
for them.

All randomness comes from NumPy's PCG64 (``numpy.random.default_rng(seed)``)
in a fixed draw order, so every array is reproducible from its seed and can
be hashed.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

DIM = 128
NORM = 512.0


def desc(rng: np.random.Generator, n: int) -> np.ndarray:
    """n fresh descriptors: |N(0,1)| per component, L2 norm 512, rint, clamp."""
    z = np.abs(rng.standard_normal((n, DIM)))
    if n:
        z *= NORM / np.linalg.norm(z, axis=1, keepdims=True)
    return np.clip(np.rint(z), 0, 255).astype(np.uint8)


def noisy(rng: np.random.Generator, x: np.ndarray, k: int) -> np.ndarray:
    """Copy of x with independent uniform integer noise in [-k, k], clamped."""
    noise = rng.integers(-k, k + 1, size=x.shape)
    return np.clip(x.astype(np.int16) + noise, 0, 255).astype(np.uint8)


def sha256(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


@dataclass
class Pair:
    """One image pair: A (nA x 128), B (nB x 128), and the planted truth."""
    A: np.ndarray
    B: np.ndarray
    truth: np.ndarray            # int64 [m, 2]: (row of A, row of B)
    max_ratio: float = 0.8
    max_distance: float = float("inf")
    cross_check: bool = True
    name: str = ""

    def params(self) -> dict:
        return dict(max_ratio=self.max_ratio, max_distance=self.max_distance,
                    cross_check=self.cross_check)


def pair(nA: int, nB: int, frac: float, k: int, seed: int = 0) -> Pair:
    """A pair with round(frac*nA) rows of A planted (noisy) in a shuffled B.

    Draw order: A, the planted source rows, the noise of the planted copies,
    the fresh rows of B, the shuffle of B.
    """
    rng = np.random.default_rng(seed)
    A = desc(rng, nA)
    m = min(int(round(frac * nA)), nB)
    src = rng.permutation(nA)[:m]
    B = np.concatenate([noisy(rng, A[src], k), desc(rng, nB - m)], axis=0)
    perm = rng.permutation(nB)
    B = np.ascontiguousarray(B[perm])
    # row t of the unshuffled B lands at position inv[t] of the shuffled B
    inv = np.empty(nB, dtype=np.int64)
    inv[perm] = np.arange(nB)
    truth = np.stack([src.astype(np.int64), inv[:m]], axis=1) if m else \
        np.zeros((0, 2), dtype=np.int64)
    return Pair(A=A, B=B, truth=truth)


def _peaked(rng: np.random.Generator, n: int) -> np.ndarray:
    """Descriptors dominated by one component, which saturates at 255."""
    z = np.abs(rng.standard_normal((n, DIM)))
    hot = rng.integers(0, DIM, size=n)
    z[np.arange(n), hot] += 40.0
    z *= NORM / np.linalg.norm(z, axis=1, keepdims=True)
    return np.clip(np.rint(z), 0, 255).astype(np.uint8)


def edge_pair(nA: int, nB: int, n_planted: int, n_dups: int,
              all255: bool, seed: int = 0) -> Pair:
    """Tie-heavy pair: planted rows, exact duplicate B rows, degenerate rows.

    * ``n_planted`` rows of A are planted in B with +-4 noise;
    * ``n_dups`` further B rows are overwritten by exact copies of planted B
      rows, so those A rows see two equal best scores (a top-1 tie);
    * 4 all-zero rows in each of A and B (the zero floor);
    * optionally 1 all-255 row in each of A and B;
    * 2 "peaked" rows per side whose largest component clamps at 255.
    Degenerate rows are written over non-planted positions only.
    """
    rng = np.random.default_rng(seed)
    A = desc(rng, nA)
    m = min(n_planted, nB)
    src = rng.permutation(nA)[:m]
    B = np.concatenate([noisy(rng, A[src], 4), desc(rng, nB - m)], axis=0)
    perm = rng.permutation(nB)
    B = np.ascontiguousarray(B[perm])
    inv = np.empty(nB, dtype=np.int64)
    inv[perm] = np.arange(nB)
    planted_b = inv[:m]
    truth = np.stack([src.astype(np.int64), planted_b], axis=1)

    free_b = np.setdiff1d(np.arange(nB), planted_b)
    free_b = rng.permutation(free_b)
    free_a = np.setdiff1d(np.arange(nA), src)
    free_a = rng.permutation(free_a)

    nd = min(n_dups, len(free_b), m)
    dup_dst = free_b[:nd]
    dup_src = planted_b[rng.permutation(m)[:nd]]
    B[dup_dst] = B[dup_src]
    fb = free_b[nd:]

    n_zero, n_peak = 4, 2
    n255 = 1 if all255 else 0
    need = n_zero + n255 + n_peak
    if len(fb) >= need and len(free_a) >= need:
        B[fb[:n_zero]] = 0
        A[free_a[:n_zero]] = 0
        if all255:
            B[fb[n_zero]] = 255
            A[free_a[n_zero]] = 255
        o = n_zero + n255
        B[fb[o:o + n_peak]] = _peaked(rng, n_peak)
        A[free_a[o:o + n_peak]] = _peaked(rng, n_peak)
    return Pair(A=A, B=B, truth=truth)


@dataclass
class Batch:
    """An image set matched exhaustively: all pairs (m, n) with m < n."""
    images: list
    pairs: np.ndarray            # int32 [P, 2]
    truth: dict = field(default_factory=dict)   # (m, n) -> int64 [t, 2]
    max_ratio: float = 0.8
    max_distance: float = float("inf")
    cross_check: bool = True
    name: str = ""

    def params(self) -> dict:
        return dict(max_ratio=self.max_ratio, max_distance=self.max_distance,
                    cross_check=self.cross_check)


def image_set(n_images: int, n_desc: int, share: float = 0.15, k: int = 3,
              seed: int = 0) -> Batch:
    """Images whose descriptors overlap with their +-1 and +-2 neighbours.

    Each image is drawn fresh; then, for every (m, n) with n - m in {1, 2}
    in lexicographic order, round(share * n_desc) not yet used rows of m are
    copied with +-k noise over not yet used rows of n.
    """
    rng = np.random.default_rng(seed)
    images = [desc(rng, n_desc) for _ in range(n_images)]
    used = [np.zeros(n_desc, dtype=bool) for _ in range(n_images)]
    cnt = int(round(share * n_desc))
    truth = {}
    for m in range(n_images):
        for n in (m + 1, m + 2):
            if n >= n_images:
                continue
            src = rng.choice(np.flatnonzero(~used[m]), size=cnt, replace=False)
            used[m][src] = True
            dst = rng.choice(np.flatnonzero(~used[n]), size=cnt, replace=False)
            used[n][dst] = True
            images[n][dst] = noisy(rng, images[m][src], k)
            truth[(m, n)] = np.stack([src, dst], axis=1).astype(np.int64)
    pairs = np.array([(a, b) for a in range(n_images)
                      for b in range(a + 1, n_images)], dtype=np.int32)
    return Batch(images=images, pairs=pairs.reshape(-1, 2), truth=truth)


# Named workloads.  Sizes follow the matcher's use: one pair of modest size,
# one pair at 8192 x 8192 (about the 10,400 features per 4000x3000 image the
# README's survey carries), a dense 32768 x 32768 pair, an exhaustive image
# set, and tie-heavy edge cases.
WORKLOADS = {
    "pair_1000x1200": lambda: _named(pair(1000, 1200, 0.30, 3, 0),
                                     "pair_1000x1200"),
    "pair_8192x8192": lambda: _named(pair(8192, 8192, 0.20, 4, 0),
                                     "pair_8192x8192", max_distance=0.7),
    "pair_32768x32768": lambda: _named(pair(32768, 32768, 0.10, 3, 0),
                                       "pair_32768x32768"),
    "edge_8192x8192_ties": lambda: _named(
        edge_pair(8192, 8192, 1638, 410, True, 0), "edge_8192x8192_ties"),
    "edge_8192x8192_ties_no255": lambda: _named(
        edge_pair(8192, 8192, 1638, 410, False, 0),
        "edge_8192x8192_ties_no255"),
    "edge_8192x96_skinny": lambda: _named(
        edge_pair(8192, 96, 48, 5, True, 0), "edge_8192x96_skinny"),
    "edge_8192x96_skinny_no255": lambda: _named(
        edge_pair(8192, 96, 48, 5, False, 0), "edge_8192x96_skinny_no255"),
    # the feature count per image of the README's 4000x3000 survey
    # (about 10,400), with the 8192 x 8192 pair's planting and gates
    "survey_10400x10400": lambda: _named(pair(10400, 10400, 0.20, 4, 0),
                                         "survey_10400x10400", max_distance=0.7),
}


def _named(p: Pair, name: str, **kw) -> Pair:
    p.name = name
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def workload(name: str) -> Pair:
    return WORKLOADS[name]()


def exhaustive_48x8192(n_images: int = 48, n_desc: int = 8192) -> Batch:
    b = image_set(n_images, n_desc, 0.15, 3, 0)
    b.name = f"exhaustive_{n_images}x{n_desc}"
    return b
