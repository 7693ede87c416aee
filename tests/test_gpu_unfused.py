"""The unfused arm (serac_match_pair_unfused) against the CPU oracle and the
stored digests, through the C ABI.

It writes the whole score matrix, reads it back in a row pass and a column
pass and finishes like the fused path, so its lists must be byte-identical
to the oracle's on every shape: ties, ragged edges of its 128 x 256 score
blocks and 512-row column bands, both cross-check settings, lenient ratios
and the match cap.
"""
import hashlib
import json
import math
import os
import sys

import numpy as np
import pytest

import oracle
from oracle_pins import tie_heavy
from sift_descriptor_nearest_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_hashes.json")


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


def check(serac, A, B, r=0.8, d=math.inf, c=True, cap=0, label=""):
    say(f"[unfused] {label} nA={len(A)} nB={len(B)} ratio={r} dist={d} cross={c} cap={cap}")
    got = serac.match_pair_unfused(dev(A), dev(B), r, d, c, max_features=cap)
    got = got.cpu().numpy().astype(np.uint32)
    want = oracle.match_pair(A, B, r, d, c, max_features=cap)
    assert got.tobytes() == want.tobytes(), label


SHAPES = [(1, 1), (1, 300), (300, 1), (127, 255), (129, 257), (513, 511), (1029, 777),
          (600, 2100)]


@pytest.mark.parametrize("nA,nB", SHAPES, ids=[f"{a}x{b}" for a, b in SHAPES])
def test_shapes(serac, nA, nB):
    rng = np.random.default_rng(nA * 31 + nB)
    p = synth.edge_pair(nA, nB, max(1, min(nA, nB) // 3), min(nA, nB) // 10, False, nA + nB)
    T, U = tie_heavy(rng, nA), tie_heavy(rng, nB)
    for r, d, c in ((0.8, math.inf, True), (0.8, 0.7, False), (1.3, math.inf, True)):
        check(serac, p.A, p.B, r, d, c, label="planted")
        check(serac, T, U, r, d, c, label="tie-heavy")


def test_cap_and_empty(serac):
    p = synth.pair(2000, 2500, 0.3, 4, seed=2)
    for cap in (1, 700, 2500):
        check(serac, p.A, p.B, cap=cap, label=f"cap {cap}")
    e = np.zeros((0, 128), np.uint8)
    assert serac.match_pair_unfused(dev(e), dev(p.B)).shape == (0, 2)
    assert serac.match_pair_unfused(dev(p.A), dev(e)).shape == (0, 2)


def test_workload_8192_digest(serac):
    """The 8192 x 8192 workload: the oracle's stored digest, and the
    workspace holds the score matrix (4 bytes per score)."""
    with open(GOLDEN) as f:
        G = json.load(f)
    p = synth.workload("pair_8192x8192")
    ent = G["pairs"]["pair_8192x8192"]
    assert synth.sha256(p.A, p.B) == ent["inputs_sha256"]
    for key, want in ent["lists"].items():
        f = dict(x.split("=") for x in key.split(","))
        r, d = float(f["ratio"]), (math.inf if f["dist"] == "inf" else float(f["dist"]))
        got = serac.match_pair_unfused(dev(p.A), dev(p.B), r, d, f["cross"] == "1")
        got = got.cpu().numpy().astype(np.uint32)
        assert len(got) == want["count"]
        assert hashlib.sha256(got.tobytes()).hexdigest() == want["sha256"], key
    assert serac.workspace_bytes() >= 8192 * 8192 * 4


def test_past_2_31_scores(serac):
    """65536 x 65536 (2^32 scores, the arm's limit): every int32 index of S
    past 2^31 is formed in 64 bits; the list equals the fused path's, which
    the oracle pins at every size below (and by its digests at 32768^2)."""
    p = synth.pair(65536, 65536, 0.05, 4, seed=12)
    a, b = dev(p.A), dev(p.B)
    say("[unfused] 65536 x 65536")
    got = serac.match_pair_unfused(a, b, 0.8, math.inf, True).cpu().numpy()
    ref = serac.match_pair(a, b, 0.8, math.inf, True).cpu().numpy()
    assert len(got) > 3000
    assert got.tobytes() == ref.tobytes()
    # a sample of rows settled by the oracle one by one
    rows = np.linspace(0, 65535, 48).astype(np.int32)
    want = oracle.match_rows(p.A, p.B, rows, 0.8)
    have = {int(i): int(j) for i, j in got.tolist()}
    for i, j in want.items():
        assert have.get(i, -1) == j, i
    serac.release_stream()                        # give the 16 GiB back
