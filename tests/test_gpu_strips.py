"""Cross-pair reuse of A in a batch (serac_tiles_strip) against the oracle.

A batch whose pairs each fit one column group is swept in strips: one
workgroup takes a row block of an image and runs through the B sides of up
to m pairs that share it as A, publishing each pair's rows at the boundary
between two pairs' chunks.  The test hook SERAC_TEST_STRIP_PAIRS=<m> (read
at the device's set-up, so each setting runs in a fresh process) forces
strips of at most m pairs whatever the batch's size.  Under several m, with
images of mixed sizes (one-chunk and one-row images, so that boundaries fall
at every chunk, images on both sides of 8192 rows, an empty image), every
list must equal the oracle's, with and without the cross-check, with
symmetric gates and with the match cap; the profiler hook names the tile
kernel that ran, so the test knows the strips were used.  A batch with a B
side wider than one column group keeps the per-pair sweep, and without the
hook the library picks strips for a large set of small images.  The host
pipeline, whose stages are batches, is checked under forced strips too.
Through the C ABI.
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CODE = f"""
import json, math, sys
sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})
import numpy as np, torch
import oracle
import sift_descriptor_nearest_amd as serac
from sift_descriptor_nearest_amd import synth
cfg = json.loads(sys.argv[1])
rng = np.random.default_rng(cfg["seed"])
sizes = cfg["sizes"]
imgs = [synth.desc(rng, n) for n in sizes]
# shared descriptors (with a little noise) between neighbouring images
for a in range(len(imgs) - 1):
    b = a + 1
    k = min(len(imgs[a]), len(imgs[b])) // 4
    if k:
        src = rng.choice(len(imgs[a]), k, replace=False)
        dst = rng.choice(len(imgs[b]), k, replace=False)
        imgs[b][dst] = synth.noisy(rng, imgs[a][src], 3)
if cfg.get("random_pairs"):
    # a random pair list: both orders, self pairs and repeats
    n = len(imgs)
    pairs = [(int(x), int(y)) for x, y in rng.integers(0, n, size=(cfg["random_pairs"], 2))]
    pairs += pairs[:5]
else:
    pairs = [(a, b) for a in range(len(imgs)) for b in range(len(imgs))
             if a != b and (a < b or (a + b) % 3 == 0)]
    pairs += [(1, 1), (0, 2)]
dev = [torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0") for x in imgs]
for prm in cfg["params"]:
    serac.profile_start(4)
    res = serac.match_pairs(dev, pairs, **prm)
    torch.cuda.synchronize()
    _, n, _, kname = serac.profile_stop()
    assert kname.startswith(cfg["kernel"]), (kname, cfg["kernel"])
    host = serac.match_pairs_host(dev, pairs, pairs_per_stage=cfg["stage"], **prm) \
        if cfg.get("stage") else None
    for q, (a, b) in enumerate(pairs):
        want = oracle.match_pair(imgs[a], imgs[b], **prm)
        got = res[q].cpu().numpy().astype(np.uint32)
        assert got.tobytes() == want.tobytes(), (prm, a, b, len(got), len(want))
        if host is not None:
            assert host[q].tobytes() == want.tobytes(), ("host", prm, a, b)
    print("ok", kname, len(pairs), json.dumps(prm), flush=True)
"""

MIXED = [2100, 700, 1, 5000, 300, 0, 3000, 2600, 64, 1500, 257, 4100]
WIDE = [9000, 700, 1, 3000, 257, 2600]
PARAMS = [dict(max_ratio=0.8, max_distance=1e9, cross_check=True),
          dict(max_ratio=0.8, max_distance=0.7, cross_check=False),
          dict(max_ratio=1.2, max_distance=1e9, cross_check=True),
          dict(max_ratio=0.8, max_distance=1e9, cross_check=True, symmetric=True),
          dict(max_ratio=0.8, max_distance=1e9, cross_check=True, max_features=1000)]

CASES = {
    # the host pipeline as well, in stages of 7 pairs (each stage a batch
    # swept in strips)
    "m2_mixed": (dict(SERAC_TEST_STRIP_PAIRS="2"),
                 dict(seed=1, sizes=MIXED, params=PARAMS, kernel="serac_tiles_strip", stage=7)),
    "m3_wide_order": (dict(SERAC_TEST_STRIP_PAIRS="3", SERAC_TEST_WG_ORDER="977"),
                      dict(seed=2, sizes=WIDE, params=PARAMS[:2], kernel="serac_tiles_strip")),
    "m16_many": (dict(SERAC_TEST_STRIP_PAIRS="16"),
                 dict(seed=3, sizes=[300, 1200, 64, 900, 1, 2000, 513, 257, 700, 1100, 40,
                                     1800, 256, 600, 1500, 900, 2200, 128, 1000, 350],
                      params=PARAMS[:1] + PARAMS[3:4], kernel="serac_tiles_strip")),
    # no hook: the library's own choice, strips for a large set of small
    # images (80 x 512 descriptors, about 5300 pairs)
    "default_small_images": ({}, dict(seed=6, sizes=[512] * 80, params=PARAMS[:1] + PARAMS[3:4],
                                      kernel="serac_tiles_strip")),
    # seeded random sets: sizes 0..3000, a random pair list, random strip
    # lengths
    "random_a": (dict(SERAC_TEST_STRIP_PAIRS="5"),
                 dict(seed=21, sizes=[int(x) for x in
                                      np.random.default_rng(21).integers(0, 3001, 14)],
                      random_pairs=90, params=PARAMS[:2], kernel="serac_tiles_strip")),
    "random_b": (dict(SERAC_TEST_STRIP_PAIRS="11"),
                 dict(seed=22, sizes=[int(x) for x in
                                      np.random.default_rng(22).integers(0, 3001, 9)] + [1, 257],
                      random_pairs=70, params=PARAMS[2:4], kernel="serac_tiles_strip")),
    "off": (dict(SERAC_TEST_STRIP_PAIRS="1"),
            dict(seed=4, sizes=MIXED[:6], params=PARAMS[:1], kernel="serac_tiles_many")),
    "too_wide_for_strips": (dict(SERAC_TEST_STRIP_PAIRS="4"),
                            dict(seed=5, sizes=[17000, 700, 1, 3000], params=PARAMS[:1],
                                 kernel="serac_tiles_many")),
}


@pytest.mark.parametrize("case", list(CASES))
def test_strips_against_oracle(case):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    env_extra, cfg = CASES[case]
    env = {k: v for k, v in os.environ.items() if k != "SERAC_TEST_STRIP_PAIRS"}
    env.update(env_extra)
    print(f"[strips] {case} {env_extra}", flush=True)
    r = subprocess.run([sys.executable, "-u", "-c", CODE, json.dumps(cfg)], env=env,
                       capture_output=True, text=True, timeout=900)
    print(r.stdout[-3000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.count("ok ") == len(cfg["params"])
