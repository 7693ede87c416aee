"""Write oracle_hashes.json: the CPU oracle's results on every named workload.

The GPU parity tests compare the HIP path's output on these workloads with
what is stored here: the SHA-256 of each match list (uint32 pairs, ascending
row, the byte layout both sides produce) and its length, and for two pairs
the SHA-256 of the oracle's row top-2 and column-best exports.  Every stored
value comes from ``oracle/`` on inputs from the seeded generator
(``sift_descriptor_nearest_amd/synth.py``); the inputs' own SHA-256 is stored
too, so a test can tell a changed generator from a changed matcher.
SHA-256 identity of the correspondence blobs is the referee the SERAC README
uses for its two arms (section "Exactness").

Run from the repository root (about 40 minutes on 8 cores, most of it the
1128 pairs of the exhaustive 48 x 8192 batch):

    python3 tests/golden/make_oracle_hashes.py
"""
from __future__ import annotations

import hashlib
import json
import math
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from sift_descriptor_nearest_amd import synth  # noqa: E402

OUT = os.path.join(HERE, "oracle_hashes.json")

# Gate settings the parity tests run each single-pair workload under: the
# workload's own, plus (for the edge pairs) the lenient ratio that lets tied
# bests through and the cross-check switched off.
EXTRA_GATES = {
    "edge_8192x8192_ties": [(1.5, math.inf, True), (0.8, math.inf, False)],
    "edge_8192x8192_ties_no255": [(1.5, math.inf, True), (0.8, math.inf, False)],
    "edge_8192x96_skinny_no255": [(1.5, math.inf, True), (0.8, math.inf, False)],
}
# Pairs whose full top-2 exports are stored as well.
TOP2 = ("pair_8192x8192", "pair_32768x32768")


def sha(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def gate_key(r: float, d: float, c: bool) -> str:
    return f"ratio={r!r},dist={'inf' if math.isinf(d) else repr(d)},cross={int(c)}"


def main() -> None:
    t0 = time.time()
    res = {"about": "SHA-256 of the CPU oracle's outputs on the named synthetic workloads "
                    "(written by tests/golden/make_oracle_hashes.py, which calls only oracle/)",
           "pairs": {}, "batch": {}}
    for name in synth.WORKLOADS:
        p = synth.workload(name)
        prm = p.params()
        gates = [(prm["max_ratio"], prm["max_distance"], prm["cross_check"])]
        gates += EXTRA_GATES.get(name, [])
        ent = {"nA": int(p.A.shape[0]), "nB": int(p.B.shape[0]),
               "inputs_sha256": synth.sha256(p.A, p.B), "lists": {}}
        for r, d, c in gates:
            lst = oracle.match_pair(p.A, p.B, r, d, c)
            ent["lists"][gate_key(r, d, c)] = {"count": int(len(lst)), "sha256": sha(lst)}
        if name in TOP2:
            row, col = oracle.top2(p.A, p.B)
            ent["top2"] = {"row_sha256": sha(row), "col_sha256": sha(col)}
        res["pairs"][name] = ent
        print(f"{name}: {time.time() - t0:.1f} s", flush=True)

    bt = synth.exhaustive_48x8192()
    prm = bt.params()
    lists = []
    for k, (a, b) in enumerate(bt.pairs.tolist()):
        lst = oracle.match_pair(bt.images[a], bt.images[b], **prm)
        lists.append({"a": a, "b": b, "count": int(len(lst)), "sha256": sha(lst)})
        if k % 100 == 0:
            print(f"batch pair {k}/{len(bt.pairs)}: {time.time() - t0:.1f} s", flush=True)
    res["batch"][bt.name] = {
        "images": len(bt.images), "n": int(bt.images[0].shape[0]),
        "inputs_sha256": synth.sha256(*bt.images),
        "gates": gate_key(prm["max_ratio"], prm["max_distance"], prm["cross_check"]),
        "lists": lists}
    res["oracle_threads"] = oracle.max_threads()
    with open(OUT, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(f"wrote {OUT} in {time.time() - t0:.1f} s")


if __name__ == "__main__":
    main()
