"""Paths switched by the library's test hooks, each in a fresh process (the
hooks are read when a device is set up or a workspace grows), through the
C ABI, against the CPU oracle.

- SERAC_TEST_ANGLE_TABLE: every ratio and distance decision is taken from
  the host-built angle table, the path the finishing kernel falls back to
  where the device angle does not settle a gate.
- SERAC_TEST_FAIL_ALLOC: every allocation the library attempts fails; a
  call reports SERAC_ERR_OUT_OF_MEMORY without writing the caller's
  outputs, and once the variable is unset the next call succeeds.
"""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PRELUDE = f"""
import math, os, sys
sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})
import numpy as np, torch
import oracle
import sift_descriptor_nearest_amd as serac
from sift_descriptor_nearest_amd import synth
from oracle_pins import tie_heavy
def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")
def check(A, B, r=0.8, d=math.inf, c=True, label=""):
    got = serac.match_pair(dev(A), dev(B), r, d, c).cpu().numpy().astype(np.uint32)
    want = oracle.match_pair(A, B, r, d, c)
    assert got.tobytes() == want.tobytes(), label
    print("ok", label, len(got), flush=True)
"""


def run(code, env_extra, timeout=240):
    env = dict(os.environ)
    env.update(env_extra)
    r = subprocess.run([sys.executable, "-u", "-c", PRELUDE + code], env=env,
                       capture_output=True, text=True, timeout=timeout)
    print(r.stdout[-3000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return r.stdout


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_angle_slack_is_tight(gpu):
    """The device angle stays within a hair of the table's, so the
    finishing kernel settles nearly every gate without the table."""
    out = run("print('slack', serac.angle_slack())", {})
    slack = float(out.split("slack")[1].split()[0])
    assert 0.0 < slack < 1e-12, slack


def test_table_only_gates(gpu):
    """With the table deciding every gate: the workload pair, the edge pair
    (saturated and tied scores), tie-heavy data at lenient ratios."""
    code = """
assert serac.angle_slack() == math.inf
p = synth.workload("pair_8192x8192"); check(p.A, p.B, 0.8, 0.7, True, "8192 table")
p = synth.workload("edge_8192x8192_ties"); check(p.A, p.B, 1.5, math.inf, True, "edge table")
rng = np.random.default_rng(5)
A, B = tie_heavy(rng, 700), tie_heavy(rng, 900)
for r in (0.8, 1.0, 1.3):
    check(A, B, r, math.inf, True, f"tie table {r}")
    check(A, B, r, 1.2, False, f"tie table {r} nocross")
"""
    run(code, {"SERAC_TEST_ANGLE_TABLE": "1"})


def test_allocation_failure_recovers(gpu):
    """Allocation failures at device set-up and at workspace growth report
    out of memory, leave the outputs untouched, and the next call works."""
    code = """
p = synth.workload("pair_1000x1200")
a, b = dev(p.A), dev(p.B)
out = torch.full((1000, 2), -7, dtype=torch.int32, device="cuda:0")
cnt = torch.full((1,), -7, dtype=torch.int32, device="cuda:0")
def expect_oom():
    try:
        serac.match_pair_into(a, b, out, cnt, **p.params())
    except serac.SeracError as e:
        assert e.status == serac.SERAC_ERR_OUT_OF_MEMORY, e.status
    else:
        raise AssertionError("expected out of memory")
    torch.cuda.synchronize()
    assert int(cnt.item()) == -7 and int(out.min()) == -7 and int(out.max()) == -7
expect_oom()                                   # first call: device set-up fails
os.environ.pop("SERAC_TEST_FAIL_ALLOC")
check(p.A, p.B, 0.8, math.inf, True, "after set-up failure")
big = synth.pair(4096, 65537, 0.2, 4, seed=3)  # prepared sets: the workspace grows
a, b = dev(big.A), dev(big.B)
out = torch.full((4096, 2), -7, dtype=torch.int32, device="cuda:0")
os.environ["SERAC_TEST_FAIL_ALLOC"] = "1"
expect_oom()                                   # workspace growth fails
os.environ.pop("SERAC_TEST_FAIL_ALLOC")
check(big.A, big.B, 0.8, math.inf, True, "after growth failure")
imgs = [dev(x) for x in (p.A, p.B, big.A)]
os.environ["SERAC_TEST_FAIL_ALLOC"] = "1"
try:
    serac.match_pairs(imgs, [(0, 1), (2, 0)], 0.8, math.inf, True)
except serac.SeracError as e:
    assert e.status == serac.SERAC_ERR_OUT_OF_MEMORY
else:
    raise AssertionError("expected out of memory (batch)")
os.environ.pop("SERAC_TEST_FAIL_ALLOC")
res = serac.match_pairs(imgs, [(0, 1), (2, 0)], 0.8, math.inf, True)
assert res[0].cpu().numpy().astype(np.uint32).tobytes() == oracle.match_pair(p.A, p.B).tobytes()
print("ok batch after failure", flush=True)
"""
    run(code, {"SERAC_TEST_FAIL_ALLOC": "1"})


def test_release_stream(gpu):
    """Workspaces of side streams are freed by serac_release_stream and
    come back on the next call; results stay the oracle's."""
    code = """
p = synth.workload("pair_1000x1200")
a, b = dev(p.A), dev(p.B)
want = oracle.match_pair(p.A, p.B, 0.8, math.inf, True)
serac.match_pair(a, b)                        # the null stream's workspace
base = serac.workspace_bytes()
streams = [torch.cuda.Stream() for _ in range(3)]
for s in streams:
    with torch.cuda.stream(s):
        assert serac.match_pair(a, b).cpu().numpy().astype(np.uint32).tobytes() == want.tobytes()
grown = serac.workspace_bytes()
assert grown > base, (grown, base)
for s in streams:
    serac.release_stream(s.cuda_stream)
    serac.release_stream(s.cuda_stream)       # a second release is a no-op
assert serac.workspace_bytes() == base, (serac.workspace_bytes(), base)
for s in streams:                             # released entries are reused
    with torch.cuda.stream(s):
        assert serac.match_pair(a, b).cpu().numpy().astype(np.uint32).tobytes() == want.tobytes()
imgs = [a, b]
with torch.cuda.stream(streams[0]):
    r = serac.match_pairs(imgs, [(0, 1), (1, 0)])
    serac.release_stream(streams[0].cuda_stream)
    assert r[0].cpu().numpy().astype(np.uint32).tobytes() == want.tobytes()
torch.cuda.synchronize()
print("ok release", base, grown, flush=True)
"""
    run(code, {})

