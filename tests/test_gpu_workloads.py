"""Every named workload in full against the CPU oracle, through the C ABI.

The oracle's match lists for the named workloads (every pair of the
48 x 8192 exhaustive batch included) and its row top-2 / column-best
exports for the 8192 x 8192 and 32768 x 32768 pairs are stored as SHA-256
digests in tests/golden/oracle_hashes.json, written by the committed script
beside it, which calls only oracle/.  The GPU's outputs must hash to the
same values and have the same lengths: byte identity, the referee the SERAC
README uses for its two arms (section "Exactness").  The inputs' digests are
checked first, so a changed generator is told apart from a changed matcher,
and a spread of batch pairs is recomputed by the oracle live, so a stale
golden file cannot hide a difference.
"""
import hashlib
import json
import math
import os
import sys

import numpy as np
import pytest

import oracle
from sift_descriptor_nearest_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "oracle_hashes.json")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def sha(a) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def gate_key(r, d, c) -> str:
    return f"ratio={r!r},dist={'inf' if math.isinf(d) else repr(d)},cross={int(c)}"


def parse_gate(key):
    f = dict(x.split("=") for x in key.split(","))
    return float(f["ratio"]), (math.inf if f["dist"] == "inf" else float(f["dist"])), \
        bool(int(f["cross"]))


with open(GOLDEN) as _f:
    G = json.load(_f)

PAIR_CASES = [(name, key) for name, ent in G["pairs"].items() for key in ent["lists"]]


@pytest.fixture(scope="module")
def serac():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sift_descriptor_nearest_amd as s
    s.library()
    return s


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


_pairs = {}


def workload(name):
    if name not in _pairs:
        p = synth.workload(name)
        assert synth.sha256(p.A, p.B) == G["pairs"][name]["inputs_sha256"], \
            f"{name}: the generator no longer makes the inputs the oracle saw"
        _pairs.clear()
        _pairs[name] = (p, dev(p.A), dev(p.B))
    return _pairs[name]


@pytest.mark.parametrize("name,key", PAIR_CASES, ids=[f"{n}[{k}]" for n, k in PAIR_CASES])
def test_named_pair_list(serac, name, key):
    p, a, b = workload(name)
    r, d, c = parse_gate(key)
    say(f"[workload] {name} {key}")
    got = serac.match_pair(a, b, r, d, c).cpu().numpy().astype(np.uint32)
    want = G["pairs"][name]["lists"][key]
    assert len(got) == want["count"], (name, key, len(got), want["count"])
    assert sha(got) == want["sha256"], (name, key)


TOP2 = [n for n, e in G["pairs"].items() if "top2" in e]


@pytest.mark.parametrize("name", TOP2)
def test_named_pair_top2(serac, name):
    p, a, b = workload(name)
    say(f"[workload] {name} top-2 export")
    row, col = serac.top2(a, b)
    want = G["pairs"][name]["top2"]
    assert sha(row.cpu().numpy()) == want["row_sha256"], name
    assert sha(col.cpu().numpy()) == want["col_sha256"], name


BATCH = synth.exhaustive_48x8192().name
BATCH_CHUNKS = 8


@pytest.fixture(scope="module")
def batch(serac):
    bt = synth.exhaustive_48x8192()
    want = G["batch"][bt.name]
    assert synth.sha256(*bt.images) == want["inputs_sha256"], \
        "the generator no longer makes the images the oracle saw"
    imgs = [dev(x) for x in bt.images]
    pairs = bt.pairs.tolist()
    assert [[w["a"], w["b"]] for w in want["lists"]] == pairs
    r, d, c = parse_gate(want["gates"])
    say(f"[workload] {bt.name}: serac_match_pairs over {len(pairs)} pairs")
    dev_lists = [x.cpu().numpy().astype(np.uint32) for x in serac.match_pairs(imgs, pairs, r, d, c)]
    say(f"[workload] {bt.name}: serac_match_pairs_host over {len(pairs)} pairs")
    host_lists = serac.match_pairs_host(imgs, pairs, r, d, c)
    return bt, want, dev_lists, host_lists


@pytest.mark.parametrize("chunk", range(BATCH_CHUNKS))
def test_batch_every_pair(batch, chunk):
    """All 1128 lists, from serac_match_pairs and serac_match_pairs_host."""
    bt, want, dev_lists, host_lists = batch
    n = len(want["lists"])
    lo, hi = chunk * n // BATCH_CHUNKS, (chunk + 1) * n // BATCH_CHUNKS
    say(f"[workload] {bt.name}: pairs {lo}..{hi - 1}")
    for k in range(lo, hi):
        w = want["lists"][k]
        for got, how in ((dev_lists[k], "match_pairs"), (host_lists[k], "match_pairs_host")):
            assert len(got) == w["count"] and sha(got) == w["sha256"], (how, w["a"], w["b"])


def test_batch_live_oracle(batch):
    """A spread of batch pairs recomputed by the oracle now: neighbours
    sharing planted rows and distant pairs, first and last."""
    bt, want, dev_lists, host_lists = batch
    r, d, c = parse_gate(want["gates"])
    ks = sorted({0, 1, 47, 93, 500, 777, len(want["lists"]) - 1})
    for k in ks:
        a, b = want["lists"][k]["a"], want["lists"][k]["b"]
        say(f"[workload] {bt.name}: live oracle on pair ({a}, {b})")
        ref = oracle.match_pair(bt.images[a], bt.images[b], r, d, c)
        assert dev_lists[k].tobytes() == ref.tobytes(), (a, b)
        assert sha(ref) == want["lists"][k]["sha256"], ("stale golden file", a, b)
