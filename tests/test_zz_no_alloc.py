"""serac_match_pair_noalloc, the entry point that allocates nothing, through
the C ABI: its lists are byte-identical to serac_match_pair's on the same
inputs, call after call on one device (the fixed scratch keeps what the last
call left), also when the second call is smaller, when its call is replayed
from a captured HIP graph, and when every allocation the library attempts
would fail; pairs beyond its limit and calls before the device's set-up are
refused with their own status codes.
"""
import math
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from sift_descriptor_nearest_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def serac():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sift_descriptor_nearest_amd as s
    s.init()
    return s


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def existing(serac, a, b, r, d, c):
    return serac.match_pair(a, b, r, d, c).cpu().numpy()


def noalloc(serac, a, b, r, d, c):
    n = a.shape[0]
    out = torch.full((max(n, 1), 2), -7, dtype=torch.int32, device=a.device)
    cnt = torch.full((1,), -7, dtype=torch.int32, device=a.device)
    serac.match_pair_noalloc_into(a, b, out, cnt, r, d, c)
    k = int(cnt.item())
    assert 0 <= k <= n
    return out[:k].cpu().numpy()


GATES = [(0.8, math.inf, True), (0.8, 0.7, False), (1.0, math.inf, False)]


@pytest.mark.parametrize("r,d,c", GATES)
def test_two_calls_second_smaller(serac, r, d, c):
    big = synth.workload("pair_8192x8192")
    small = synth.workload("pair_1000x1200")
    A, B = dev(big.A), dev(big.B)
    a, b = dev(small.A), dev(small.B)
    say(f"[noalloc] 8192x8192 then 1000x1200, gates {r} {d} {c}")
    got_big = noalloc(serac, A, B, r, d, c)
    got_small = noalloc(serac, a, b, r, d, c)
    assert got_big.tobytes() == existing(serac, A, B, r, d, c).tobytes()
    assert got_small.tobytes() == existing(serac, a, b, r, d, c).tobytes()
    assert got_small.astype(np.uint32).tobytes() == \
        oracle.match_pair(small.A, small.B, r, d, c).tobytes()
    # and back up again: what the smaller call left does not leak
    again = noalloc(serac, A, B, r, d, c)
    assert again.tobytes() == got_big.tobytes()


def test_shapes_at_the_limits(serac):
    """Empty sets, a skinny ragged pair, and 16384 x 16384 (the largest
    square pair the fixed scratch takes on every gfx950 part)."""
    rng = np.random.default_rng(11)
    e = dev(np.zeros((0, 128), np.uint8))
    x = dev(synth.pair(300, 10, 0.2, 4, seed=2).A)
    for a, b in ((e, x), (x, e)):
        out = torch.full((max(a.shape[0], 1), 2), -7, dtype=torch.int32, device="cuda:0")
        cnt = torch.full((1,), -7, dtype=torch.int32, device="cuda:0")
        serac.match_pair_noalloc_into(a, b, out, cnt)
        assert int(cnt.item()) == 0
    p = synth.workload("edge_8192x96_skinny")
    a, b = dev(p.A), dev(p.B)
    say("[noalloc] 8192x96 skinny")
    assert noalloc(serac, a, b, 0.8, math.inf, True).tobytes() == \
        existing(serac, a, b, 0.8, math.inf, True).tobytes()
    big = synth.pair(16384, 16384, 0.2, 4, seed=4)
    a, b = dev(big.A), dev(big.B)
    say("[noalloc] 16384x16384")
    for c in (True, False):
        assert noalloc(serac, a, b, 0.8, math.inf, c).tobytes() == \
            existing(serac, a, b, 0.8, math.inf, c).tobytes()
    say("[noalloc] 8192x32768 refused")
    wide = dev(rng.integers(0, 64, size=(32768, 128), dtype=np.uint8))
    a8 = dev(synth.workload("pair_8192x8192").A)
    out = torch.empty((8192, 2), dtype=torch.int32, device="cuda:0")
    cnt = torch.empty(1, dtype=torch.int32, device="cuda:0")
    with pytest.raises(serac.SeracError) as ei:
        serac.match_pair_noalloc_into(a8, wide, out, cnt)
    assert ei.value.status == serac.SERAC_ERR_TOO_LARGE


def test_graph_replay(serac):
    """A captured call replayed three times, with eager calls of both entry
    points and clears of its outputs between the replays: each replay gives
    the eager list (the accumulators are zero again at the end of a call)."""
    p = synth.workload("pair_8192x8192")
    q = synth.workload("pair_1000x1200")
    a, b = dev(p.A), dev(p.B)
    qa, qb = dev(q.A), dev(q.B)
    want = existing(serac, a, b, 0.8, math.inf, True)
    out = torch.full((8192, 2), -7, dtype=torch.int32, device="cuda:0")
    cnt = torch.full((1,), -7, dtype=torch.int32, device="cuda:0")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                        # warm-up off the capture
        serac.match_pair_noalloc_into(a, b, out, cnt)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("[noalloc] capture")
    with torch.cuda.graph(g):
        serac.match_pair_noalloc_into(a, b, out, cnt)
    torch.cuda.synchronize()
    for k in range(3):
        out.fill_(-7)
        cnt.fill_(-7)
        torch.cuda.synchronize()
        say(f"[noalloc] replay {k}")
        g.replay()
        torch.cuda.synchronize()
        n = int(cnt.item())
        assert out[:n].cpu().numpy().tobytes() == want.tobytes(), k
        # eager work on the same scratch between replays
        assert noalloc(serac, qa, qb, 0.8, math.inf, True).tobytes() == \
            existing(serac, qa, qb, 0.8, math.inf, True).tobytes()
        torch.cuda.synchronize()
    del g


PRELUDE = f"""
import math, os, sys
sys.path.insert(0, {ROOT!r})
import numpy as np, torch
import sift_descriptor_nearest_amd as serac
from sift_descriptor_nearest_amd import synth
def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")
def call(fn, a, b):
    out = torch.full((a.shape[0], 2), -7, dtype=torch.int32, device="cuda:0")
    cnt = torch.full((1,), -7, dtype=torch.int32, device="cuda:0")
    fn(a, b, out, cnt)
    n = int(cnt.item())
    return out[:n].cpu().numpy()
"""


def run(code, env_extra=None, timeout=240):
    env = dict(os.environ)
    env.update(env_extra or {})
    r = subprocess.run([sys.executable, "-u", "-c", PRELUDE + code], env=env,
                       capture_output=True, text=True, timeout=timeout)
    print(r.stdout[-3000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0, r.stderr[-3000:]


def test_refused_before_setup(serac):
    """In a fresh process the first call, before any set-up, is refused
    (it would have to allocate); after serac_init it runs."""
    run("""
p = synth.workload("pair_1000x1200"); a, b = dev(p.A), dev(p.B)
try:
    call(serac.match_pair_noalloc_into, a, b)
except serac.SeracError as e:
    assert e.status == serac.SERAC_ERR_NOT_INITIALIZED, e.status
else:
    raise AssertionError("expected SERAC_ERR_NOT_INITIALIZED")
serac.init()
got = call(serac.match_pair_noalloc_into, a, b)
assert got.tobytes() == call(serac.match_pair_into, a, b).tobytes()
print("ok", len(got), flush=True)
""")


def test_runs_when_every_allocation_fails(serac):
    """With the library's allocation hook failing every attempt, the
    allocating entry point reports out of memory where it must grow, and
    the non-allocating one still gives its list."""
    run("""
serac.init()
p = synth.workload("pair_8192x8192"); a, b = dev(p.A), dev(p.B)
q = synth.workload("pair_1000x1200"); qa, qb = dev(q.A), dev(q.B)
want, want_q = call(serac.match_pair_into, a, b), call(serac.match_pair_into, qa, qb)
os.environ["SERAC_TEST_FAIL_ALLOC"] = "1"
s = torch.cuda.Stream()                  # a new stream: the allocating path needs a workspace
with torch.cuda.stream(s):
    try:
        call(serac.match_pair_into, a, b)
    except serac.SeracError as e:
        assert e.status == serac.SERAC_ERR_OUT_OF_MEMORY, e.status
    else:
        raise AssertionError("expected out of memory")
    assert call(serac.match_pair_noalloc_into, a, b).tobytes() == want.tobytes()
    assert call(serac.match_pair_noalloc_into, qa, qb).tobytes() == want_q.tobytes()
print("ok", flush=True)
""")
