"""Benchmark: int8 TOPS and ms/pair of the fused matcher on one MI355X.

One step is one call of serac_match_pair on a 8192 x 8192 pair of 128-d
uint8 descriptors (20% planted with +-4 noise, ratio 0.8, max distance 0.7
rad, cross-check on): at this size two kernels, the fused tile kernel
(which converts the raw descriptors itself) and the finishing kernel
(gates, cross-check, ordered output).
Inputs are resident in HBM before the timed region; outputs are
preallocated, poisoned before the warm-up, and the last step's match list
is compared byte for byte with the CPU oracle after the timed region.  The
2000 warm-up steps (~40 ms) bring the device to its steady clock, which
it reaches only after ~1000 back-to-back steps.

Prints one JSON line.  `value` and `ms_per_step` come from the timed region.
`roofline` is for the dominant kernel (the tile kernel, named by the
library): its mean and median launch duration, from HIP start/stop events
attached to its dispatches on the launch stream (hipExtLaunchKernel): one
launch in PROFILE_EVERY inside the timed region (events on every dispatch
would slow the enqueueing host enough to lower the step rate), and when
that is fewer than MIN_TIMED_LAUNCHES (a short run), back-to-back steps
right after the timed region with every launch timed, up to that many.  Under rocprofv3 these readings are not meaningful (the profiler
takes over the dispatch timestamps), so there the profiler's own kernel
trace is the measurement.  `traffic` is the HBM bytes per launch from the
committed counter runs of this command, null once the device code has changed.
`cpu_baseline` is the oracle on this host's cores, timed on a bounded
number of full-pair runs, with the CPU model and the single-thread time of
the 1000 x 1200 and 8192 x 8192 pairs.  `sha256` holds the inputs' and the
match lists' digests (the SERAC README's referee for identical outputs).

`--host-pipeline` measures instead the exhaustive 48-image batch (1128
pairs of 8192 x 8192) delivered to host memory by serac_match_pairs_host,
per pair, at several stage sizes: one stage of all pairs is the unpipelined
order (match everything, then copy), smaller stages overlap the copies and
the host's unpacking with the matching of later stages.  The device-only
batch (serac_match_pairs, results left on the device) is timed beside it.

`--configs` times every named workload (the parity configurations, the
README survey's image shape 10400 x 10400, and the exhaustive batch), one
JSON line each, with every match list (all 1128 of the batch) checked
against the oracle's through the SHA-256 values the oracle wrote to
tests/golden/oracle_hashes.json.

`--mfma-ceiling` measures the int8 MFMA ceiling of the device, the shader
clock it runs at, and what vector instructions issued beside MFMAs cost
(libserac_probe.so), the figures the sweep's bound is derived from.

`--unfused` times the fused matcher against the unfused arm (the score
matrix written to device memory, then row and column passes) on the 8192^2
and 32768^2 workloads, with each arm's workspace: the analogue of the SERAC
README's kernel-time and memory tables.

`--clock-ramp` records the shader clock and the step time against the
number of back-to-back steps from a cold start (why the default run warms
up for 2000 steps).

`--f1-probe` bounds what reusing staged A tiles across the pairs of a batch
could save: the fixed per-workgroup part of batch sweeps of 1 to 32 chunks.

`--strips` times exhaustive image sets of 512 to 10400 descriptors per
image with the pairs swept one by one, in strips of up to 16 pairs that
share their A image (cross-pair reuse), and as the library chooses, each in
a child process (the library reads the setting at start-up), and checks
that the lists are identical.

`--copy-probe MIB` and `--write-traffic DIR` make the traffic record: the
first runs a plain copy of known size for the counter scales, the second
(on any host) turns four rocprofv3 FETCH_SIZE / WRITE_SIZE runs into
profiles/traffic_tiles_pair_8192x8192.json.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, published
PEAK_CLOCK_GHZ = 2.4         # the clock that published peak is quoted at
# Tile-kernel launches per event-timed one in long runs: the event handling
# slows the enqueueing host, and at 1 in 8 it cost ~0.15 us per step (958
# against 966 TOPS at 1 in 32 or 1 in 128, same box); the kernel time read
# is the same.  Short runs time every launch (see sample_every).
PROFILE_EVERY = 32
MIN_TIMED_LAUNCHES = 16
# The headline workload's metric, worded as the benchmark's own definition.
METRIC_8192 = "int8 TOPS and ms/pair, 8192\u00d78192\u00d7128 uint8 pair; % of MFMA int8 peak"
TRAFFIC = os.path.join(ROOT, "profiles", "traffic_tiles_pair_8192x8192.json")


def kernel_sha() -> str:
    """sha256 of the device code the benchmark runs: the gfx950 code object
    embedded in the library (its .hip_fatbin section).  Host-only and
    comment changes leave it alone; any change to a kernel or to the device
    compilation changes it."""
    import struct
    from sift_descriptor_nearest_amd import LIB_PATH
    with open(LIB_PATH, "rb") as f:
        d = f.read()
    if d[:4] != b"\x7fELF" or d[4] != 2:
        raise RuntimeError(f"{LIB_PATH} is not a 64-bit ELF library")
    shoff = struct.unpack_from("<Q", d, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", d, 0x3A)

    def header(i):
        return struct.unpack_from("<IIQQQQ", d, shoff + i * shentsize)

    names = header(shstrndx)[4]
    for i in range(shnum):
        name, _, _, _, off, size = header(i)
        end = d.index(b"\0", names + name)
        if d[names + name:end] == b".hip_fatbin":
            return hashlib.sha256(d[off:off + size]).hexdigest()
    raise RuntimeError(f"{LIB_PATH} holds no .hip_fatbin section")


def measured_traffic():
    """(HBM bytes per tile-kernel launch, where they come from) from the
    committed counter runs of this benchmark's command, or (None, reason)
    when the kernel source or its build flags have changed since they were
    taken."""
    try:
        with open(TRAFFIC) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None, "no committed counter run"
    if t.get("kernel_sha256") != kernel_sha():
        return None, "kernel changed since the committed counter run"
    return t.get("bytes_per_launch"), (
        f"committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs ({os.path.relpath(TRAFFIC, ROOT)}, "
        f"kernel sha256 {t['kernel_sha256'][:16]}..., commands in that file)")


TRAFFIC_RUNS = ("fetch", "write", "copy_fetch", "copy_write")
COPY_PROBE_MIB = 256


def counter_rows(folder: str):
    """(kernel name, counter name, value) of every dispatch in the
    rocprofv3 --pmc CSV output under `folder`."""
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(folder, "**", "*counter_collection.csv"),
                                 recursive=True)):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                rows.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no rocprofv3 counter CSV under {folder}")
    return rows


def write_traffic(folder: str, kernel: str, workload: str) -> int:
    """Writes the traffic record from four rocprofv3 --pmc runs kept under
    folder/{fetch,write,copy_fetch,copy_write}: FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch) of `kernel` in this benchmark, and of the copy
    probe, whose bytes are known and give each counter's scale."""
    def per_dispatch(run, counter, match, largest=None):
        v = [x for k, c, x in counter_rows(os.path.join(folder, run))
             if c == counter and match in k]
        if largest:
            v = sorted(v)[-largest:]
        if not v:
            raise SystemExit(f"{run}: no {counter} of a kernel named like {match!r}")
        return sum(v) / len(v), len(v)

    fetch, nf = per_dispatch("fetch", "FETCH_SIZE", kernel)
    write, nw = per_dispatch("write", "WRITE_SIZE", kernel)
    copy_bytes = COPY_PROBE_MIB << 20
    cf, _ = per_dispatch("copy_fetch", "FETCH_SIZE", "copyBuffer", largest=10)
    cw, _ = per_dispatch("copy_write", "WRITE_SIZE", "copyBuffer", largest=10)
    fs, ws = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    bench = "python3 <repo>/bench.py --gpus 1 --steps 20 --warmup 5 --no-cpu-baseline"
    probe = f"python3 <repo>/bench.py --copy-probe {COPY_PROBE_MIB}"
    rec = {
        "kernel": kernel, "workload": workload, "kernel_sha256": kernel_sha(),
        "fetch_size_kib_per_launch": round(fetch, 1), "write_size_kib_per_launch": round(write, 1),
        "dispatches": [nf, nw],
        "copy_probe_bytes": copy_bytes, "copy_probe_fetch_size_kib": round(cf, 4),
        "copy_probe_write_size_kib": round(cw, 4),
        "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
        "bytes_per_launch": int(round(fetch * 1024 * fs + write * 1024 * ws)),
        "commands": [
            "cd /tmp && export TMPDIR=/tmp",
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/fetch -o run -- {bench}",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/write -o run -- {bench}",
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/copy_fetch -o run -- {probe}",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/copy_write -o run -- {probe}",
            f"python3 <repo>/bench.py --write-traffic <out>",
        ],
        "note": "per-dispatch means over the tile kernel's dispatches in each bench run; "
                "the copy probe is 10 copies of a 256 MiB buffer (the runtime's copy kernel), "
                "its counters against the bytes it moves give the scales",
    }
    with open(TRAFFIC, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec), flush=True)
    return 0


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(p, budget_s: float):
    """The oracle as it stands on this host: full matches of the workload on
    all cores for about budget_s, plus single-thread times of the 1000 x 1200
    and 8192 x 8192 pairs."""
    import oracle
    from sift_descriptor_nearest_amd import synth
    cores = oracle.max_threads()
    ops = 2.0 * 128 * p.A.shape[0] * p.B.shape[0]
    runs, t0 = 0, time.perf_counter()
    while True:
        ref = oracle.match_pair(p.A, p.B, **p.params())
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or runs >= 200:
            break
    single = {}
    for name in ("pair_1000x1200", "pair_8192x8192"):
        q = p if name == p.name else synth.workload(name)
        t1 = time.perf_counter()
        oracle.match_pair(q.A, q.B, **q.params(), nthreads=1)
        single[name] = round(time.perf_counter() - t1, 3)
    # (the oracle's thread count sticks: restore it)
    oracle.match_pair(p.A[:1], p.B[:1], nthreads=cores)
    return ref, {"value": round(ops * runs / el / 1e12, 4), "unit": "TOPS",
                 "cores": cores, "kind": "oracle",
                 "sample": f"{runs} full {p.name} matches (oracle_match_pair, OpenMP, "
                           f"{el:.1f} s)",
                 "cpu_model": cpu_model(), "single_thread_s": single}


def list_sha(x) -> str:
    import numpy as np
    return hashlib.sha256(np.ascontiguousarray(x).tobytes()).hexdigest()


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5000)
    # the device reaches its steady clock after ~1000 back-to-back steps
    # (measured: 920 TOPS after 100 warm-up steps, 952-958 after 1000-5000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default="pair_8192x8192")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-every", type=int, default=PROFILE_EVERY, metavar="K",
                    help="attach timing events to one tile-kernel launch in K (at least "
                         f"{MIN_TIMED_LAUNCHES} launches are timed)")
    ap.add_argument("--host-pipeline", action="store_true",
                    help="instead of the benchmark, time the exhaustive batch delivered to "
                         "host memory at several stage sizes (one JSON line)")
    ap.add_argument("--configs", action="store_true",
                    help="instead of the benchmark, time every named workload (one JSON "
                         "line each)")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="instead of the benchmark, measure the int8 MFMA ceiling, the "
                         "shader clock and the issue cost of vector instructions beside "
                         "MFMAs (one JSON line)")
    ap.add_argument("--unfused", action="store_true",
                    help="instead of the benchmark, time the fused matcher against the unfused "
                         "arm (score matrix in memory) and report each arm's workspace")
    ap.add_argument("--clock-ramp", action="store_true",
                    help="instead of the benchmark, record the shader clock and the step time "
                         "against the number of back-to-back steps from a cold start")
    ap.add_argument("--f1-probe", action="store_true",
                    help="instead of the benchmark, bound what cross-pair reuse of A tiles in "
                         "a batch could save (one JSON line)")
    ap.add_argument("--strips", action="store_true",
                    help="instead of the benchmark, time exhaustive image sets of several "
                         "image sizes with pairs swept one by one, in strips of pairs that "
                         "share their A image, and as the library chooses (one JSON line)")
    ap.add_argument("--strips-child", type=int, default=0, metavar="REPS",
                    help=argparse.SUPPRESS)
    ap.add_argument("--write-traffic", metavar="DIR",
                    help="on any host: write the traffic record from the four rocprofv3 "
                         "--pmc runs under DIR/{fetch,write,copy_fetch,copy_write}")
    ap.add_argument("--traffic-kernel", default="serac_tiles_fused<true, true>",
                    help="the kernel --write-traffic reads (the bench line's roofline kernel)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, copy a MIB-MiB device buffer 10 times "
                         "(a plain copy kernel of known traffic, for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.write_traffic:
        return write_traffic(args.write_traffic, args.traffic_kernel, args.workload)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); pairs are independent, so several GPUs would "
              "each match their own share of the pair list", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be at least 1 and --warmup at least 0", file=sys.stderr)
        return 2
    if args.strips:
        return strips_compare()

    import numpy as np
    import torch

    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 10}), flush=True)
        return 0

    import sift_descriptor_nearest_amd as serac
    from sift_descriptor_nearest_amd import synth

    serac.library()
    if args.mfma_ceiling:
        return mfma_ceiling(serac)
    if args.host_pipeline:
        return host_pipeline(serac, synth, torch, np)
    if args.configs:
        return all_configs(serac, synth, torch, np)
    if args.f1_probe:
        return f1_probe(serac, synth, torch, np)
    if args.clock_ramp:
        return clock_ramp(serac, synth, torch, np)
    if args.unfused:
        return unfused_arm(serac, synth, torch, np)
    if args.strips_child:
        return strips_child(serac, synth, torch, np, args.strips_child)
    dev = torch.device("cuda:0")
    p = synth.workload(args.workload)
    nA, nB = p.A.shape[0], p.B.shape[0]
    a = torch.from_numpy(p.A).to(dev)
    b = torch.from_numpy(p.B).to(dev)
    out = torch.full((nA, 2), -1, dtype=torch.int32, device=dev)
    cnt = torch.full((1,), -1, dtype=torch.int32, device=dev)
    prm = p.params()
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        serac.match_pair_into(a, b, out, cnt, **prm)
    torch.cuda.synchronize()

    # the dominant kernel's launch duration, live in the timed region: HIP
    # events attached to one tile-kernel dispatch in `every` on the launch
    # stream (timing more of them slows the enqueueing host, which would
    # lower the step rate measured here)
    every = max(1, args.profile_every)
    serac.profile_start(args.steps // every + 1, every)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        serac.match_pair_into(a, b, out, cnt, **prm)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    _, in_region, per, kname = serac.profile_stop()
    got = out[: int(cnt.item())].cpu().numpy().astype(np.uint32)
    # a short run times too few launches that way: it is followed by
    # back-to-back steps with every launch timed, up to MIN_TIMED_LAUNCHES
    extra = max(0, MIN_TIMED_LAUNCHES - in_region)
    if extra:
        serac.profile_start(extra, 1)
        for _ in range(extra):
            serac.match_pair_into(a, b, out, cnt, **prm)
        torch.cuda.synchronize()
        _, n2, per2, kname2 = serac.profile_stop()
        per = per + per2
        kname = kname2 if in_region == 0 else (kname if kname == kname2 else "mixed")
    launches = len(per)
    kms = float(sum(per))

    ops = 2.0 * 128 * nA * nB
    wall = t1 - t0
    ms_step = wall / args.steps * 1e3
    value = ops * args.steps / wall / 1e12
    roof = {"bound": "mfma", "peak": PEAK_INT8_TOPS, "unit": "TOP/s", "kernel": kname,
            "launches": launches, "launches_in_timed_region": in_region, "every": every}
    if launches:
        k_s = kms / launches / 1e3
        med_s = float(np.median(per)) / 1e3
        achieved = ops / k_s / 1e12
        roof.update({"achieved": round(achieved, 3), "frac": round(achieved / PEAK_INT8_TOPS, 4),
                     "kernel_us": round(k_s * 1e6, 3), "kernel_us_median": round(med_s * 1e6, 3),
                     "frac_median": round(ops / med_s / 1e12 / PEAK_INT8_TOPS, 4)})
    else:
        roof.update({"achieved": None, "frac": None})
    traffic, source = measured_traffic()
    roof["traffic"] = traffic
    roof["traffic_source"] = source
    metric = METRIC_8192 if (nA, nB) == (8192, 8192) else \
        f"int8 TOPS and ms/pair, {nA}\u00d7{nB}\u00d7128 uint8 pair; % of MFMA int8 peak"
    line = {
        "metric": metric,
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": p.name, "nA": nA, "nB": nB, "dim": 128,
                   "max_ratio": prm["max_ratio"], "max_distance": prm["max_distance"],
                   "cross_check": prm["cross_check"], "seed": 0},
        "pct_of_peak": round(100.0 * value / PEAK_INT8_TOPS, 2),
        "roofline": roof,
        "matches": int(len(got)),
        "sha256": {"inputs": synth.sha256(p.A, p.B), "gpu_list": list_sha(got)},
    }
    if not args.no_cpu_baseline:
        ref, cpu = cpu_baseline(p, args.cpu_seconds)
        line["cpu_baseline"] = cpu
        line["sha256"]["oracle_list"] = list_sha(ref)
        line["identical_to_oracle"] = bool(ref.tobytes() == got.tobytes())
    print(json.dumps(line), flush=True)
    if "identical_to_oracle" in line and not line["identical_to_oracle"]:
        return 1
    return 0


def mfma_ceiling(serac) -> int:
    """The matrix-core ceiling and the issue cost of vector instructions
    beside MFMAs (libserac_probe.so), with the shader clock they ran at."""
    iters = 20000
    res = {}
    for waves, blocks in ((1, 256), (2, 512)):
        for nv in (0, 4, 8, 12, 16):
            ms, tops, ghz = serac.probe_mfma(blocks, iters, nv)
            # SIMD cycles per MFMA: waves per SIMD * rounds * 4 MFMAs per round
            cyc = ms * 1e-3 * ghz * 1e9 / (waves * iters * 4.0)
            res[f"waves{waves}_nv{nv}"] = {"tops": round(tops, 1), "ghz": round(ghz, 3),
                                           "cycles_per_mfma": round(cyc, 2)}
    base = res["waves2_nv0"]
    line = {
        "metric": "int8 MFMA ceiling, back-to-back v_mfma_i32_32x32x32_i8",
        "value": base["tops"], "unit": "TOPS", "higher_is_better": True, "n_gpus": 1,
        "shader_clock_ghz": base["ghz"],
        "peak_published": PEAK_INT8_TOPS,
        "peak_at_observed_clock": round(PEAK_INT8_TOPS * base["ghz"] / PEAK_CLOCK_GHZ, 1),
        "frac_of_published": round(base["tops"] / PEAK_INT8_TOPS, 4),
        "issue_model": res,
        "note": "nv = independent v_max3_u32 issued after each MFMA; cycles_per_mfma is "
                "SIMD cycles per MFMA at the observed clock",
    }
    print(json.dumps(line), flush=True)
    return 0


def warm_device(serac, synth, torch, steps: int = 2000) -> None:
    """Back-to-back 8192 x 8192 matches until the device holds its steady
    clock (~1000 steps, measured)."""
    p = synth.workload("pair_8192x8192")
    a = torch.from_numpy(p.A).to("cuda:0")
    b = torch.from_numpy(p.B).to("cuda:0")
    out = torch.empty((p.A.shape[0], 2), dtype=torch.int32, device="cuda:0")
    cnt = torch.empty(1, dtype=torch.int32, device="cuda:0")
    for _ in range(steps):
        serac.match_pair_into(a, b, out, cnt, **p.params())
    torch.cuda.synchronize()


GOLDEN = os.path.join(ROOT, "tests", "golden", "oracle_hashes.json")


def golden():
    """The CPU oracle's results on the named workloads, as SHA-256 of each
    match list (tests/golden/oracle_hashes.json, written by the committed
    script beside it from the oracle alone)."""
    with open(GOLDEN) as f:
        return json.load(f)


def gate_key(r, d, c) -> str:
    return f"ratio={r!r},dist={'inf' if math.isinf(d) else repr(d)},cross={int(c)}"


def all_configs(serac, synth, torch, np) -> int:
    """Per-call device time of every named workload, each match list checked
    against the oracle's (by SHA-256, every pair of the batch included)."""
    G = golden()
    ok = True
    warm_device(serac, synth, torch)

    def emit(name, nA, nB, us, ops, got_ok, matches, **extra):
        line = {"config": name, "nA": nA, "nB": nB, "us_per_call": round(us, 3),
                "tops": round(ops / us / 1e6, 2),
                "pct_of_peak": round(100.0 * ops / us / 1e6 / PEAK_INT8_TOPS, 2),
                "matches": matches, "identical_to_oracle": got_ok, **extra}
        print(json.dumps(line), flush=True)

    for name in synth.WORKLOADS:
        p = synth.workload(name)
        prm = p.params()
        want = G["pairs"][name]
        if want["inputs_sha256"] != synth.sha256(p.A, p.B):
            raise RuntimeError(f"{name}: generated inputs differ from the ones the oracle saw")
        want = want["lists"][gate_key(prm["max_ratio"], prm["max_distance"], prm["cross_check"])]
        nA, nB = p.A.shape[0], p.B.shape[0]
        a = torch.from_numpy(p.A).to("cuda:0")
        b = torch.from_numpy(p.B).to("cuda:0")
        out = torch.empty((nA, 2), dtype=torch.int32, device="cuda:0")
        cnt = torch.empty(1, dtype=torch.int32, device="cuda:0")
        ops = 2.0 * 128 * nA * nB
        reps = int(min(2000, max(20, 2e-1 / max(ops / 1.5e15, 1e-6))))
        for _ in range(20):
            serac.match_pair_into(a, b, out, cnt, **prm)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            serac.match_pair_into(a, b, out, cnt, **prm)
        e1.record()
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / reps
        got = out[: int(cnt.item())].cpu().numpy().astype(np.uint32)
        same = bool(list_sha(got) == want["sha256"] and len(got) == want["count"])
        ok = ok and same
        # the dominant kernel's own time: 16 further calls, each tile launch
        # event-timed
        serac.profile_start(16, 1)
        for _ in range(16):
            serac.match_pair_into(a, b, out, cnt, **prm)
        torch.cuda.synchronize()
        _, n, per, kname = serac.profile_stop()
        extra = {"tile_kernel": kname, "tile_us_mean": round(1e3 * float(np.mean(per)), 3),
                 "tile_us_median": round(1e3 * float(np.median(per)), 3), "tile_launches": n,
                 "tile_frac": round(ops / (1e-3 * float(np.mean(per))) / 1e12 / PEAK_INT8_TOPS, 4)}
        if nA * nB <= 8192 * 8192:
            # the oracle's time for the same list, on this host's cores
            import oracle
            t0 = time.perf_counter()
            ref = oracle.match_pair(p.A, p.B, **prm)
            extra.update({"oracle_s": round(time.perf_counter() - t0, 3),
                          "oracle_cores": oracle.max_threads(),
                          "oracle_identical": bool(ref.tobytes() == got.tobytes())})
            ok = ok and extra["oracle_identical"]
        emit(name, nA, nB, us, ops, same, int(len(got)), calls=reps,
             inputs_sha256=synth.sha256(p.A, p.B), list_sha256=list_sha(got), **extra, **prm)

    bt = synth.exhaustive_48x8192()
    want = G["batch"][bt.name]
    if want["inputs_sha256"] != synth.sha256(*bt.images):
        raise RuntimeError(f"{bt.name}: generated inputs differ from the ones the oracle saw")
    imgs = [torch.from_numpy(x).to("cuda:0") for x in bt.images]
    bp = bt.pairs.tolist()
    res = serac.match_pairs(imgs, bp, **bt.params())
    torch.cuda.synchronize()
    best = math.inf
    for _ in range(5):
        t0 = time.perf_counter()
        res = serac.match_pairs(imgs, bp, **bt.params())
        torch.cuda.synchronize()
        best = min(best, time.perf_counter() - t0)
    ops = sum(2.0 * 128 * bt.images[x].shape[0] * bt.images[y].shape[0] for x, y in bp)
    same = all(list_sha(r.cpu().numpy().astype(np.uint32)) == w["sha256"]
               for r, w in zip(res, want["lists"]))
    ok = ok and same
    emit(bt.name, 8192, 8192, best * 1e6 / len(bp), ops / len(bp), bool(same),
         int(sum(len(r) for r in res)), pairs=len(bp), timing="per pair, best of 5 calls",
         oracle_pairs_checked=len(bp))
    return 0 if ok else 1


def host_pipeline(serac, synth, torch, np, reps: int = 5) -> int:
    """Stage-level time per pair of the exhaustive batch, to host memory."""
    bt = synth.exhaustive_48x8192()
    imgs = [torch.from_numpy(x).to("cuda:0") for x in bt.images]
    pairs = bt.pairs.tolist()
    prm = bt.params()
    P = len(pairs)
    warm_device(serac, synth, torch)

    def timed(fn):
        fn()                                   # warm-up (allocations, pinned memory)
        torch.cuda.synchronize()
        best = math.inf
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            best = min(best, time.perf_counter() - t0)
        return best * 1e3 / P

    dev_ms = timed(lambda: serac.match_pairs(imgs, pairs, **prm))
    stages = {}
    ref = None
    for per in (P, 256, 64, 16):
        stages[per] = timed(lambda: serac.match_pairs_host(imgs, pairs, pairs_per_stage=per, **prm))
        got = serac.match_pairs_host(imgs, pairs, pairs_per_stage=per, **prm)
        if ref is None:
            ref = got
        elif any(a.tobytes() != b.tobytes() for a, b in zip(ref, got)):
            print("stage sizes disagree", file=sys.stderr)
            return 1
    best = min(stages, key=stages.get)
    line = {
        "metric": "ms/pair to host memory, exhaustive 48 x 8192 (1128 pairs)",
        "value": round(stages[best], 5), "unit": "ms/pair", "higher_is_better": False,
        "n_gpus": 1, "reps": reps, "timing": "best of reps, wall clock, whole call",
        "data": "synthetic",
        "config": {"workload": bt.name, "pairs": P, "pairs_per_stage": best},
        "stages_ms_per_pair": {str(k): round(v, 5) for k, v in stages.items()},
        "unpipelined_ms_per_pair": round(stages[P], 5),
        "device_only_ms_per_pair": round(dev_ms, 5),
        "matches": int(sum(len(x) for x in ref)),
    }
    print(json.dumps(line), flush=True)
    return 0


def unfused_arm(serac, synth, torch, np, reps: int = 20) -> int:
    """The fused matcher against the unfused arm (score matrix in device
    memory, then row and column passes): time per pair and device memory of
    each, on the 8192 x 8192 and 32768 x 32768 workloads, lists compared.
    Each arm runs on a stream of its own, so each has its own workspace;
    its size after the first call is the arm's device memory (the inputs
    and the output list aside)."""
    warm_device(serac, synth, torch)
    res = {}
    for name in ("pair_8192x8192", "pair_32768x32768"):
        p = synth.workload(name)
        prm = p.params()
        a = torch.from_numpy(p.A).to("cuda:0")
        b = torch.from_numpy(p.B).to("cuda:0")
        nA = p.A.shape[0]
        arms = {}
        lists = {}
        for arm, fn in (("fused", serac.match_pair_into),
                        ("unfused", serac.match_pair_unfused_into)):
            st = torch.cuda.Stream()
            out = torch.empty((nA, 2), dtype=torch.int32, device="cuda:0")
            cnt = torch.empty(1, dtype=torch.int32, device="cuda:0")
            with torch.cuda.stream(st):
                ws0 = serac.workspace_bytes()
                fn(a, b, out, cnt, **prm)
                st.synchronize()
                ws = serac.workspace_bytes() - ws0
                n = reps if nA <= 8192 else max(3, reps // 4)
                t0 = time.perf_counter()
                for _ in range(n):
                    fn(a, b, out, cnt, **prm)
                st.synchronize()
                us = (time.perf_counter() - t0) / n * 1e6
            lists[arm] = out[: int(cnt.item())].cpu().numpy().tobytes()
            arms[arm] = {"us_per_pair": round(us, 2), "workspace_mib": round(ws / 2**20, 2)}
        res[name] = {**arms, "speedup": round(arms["unfused"]["us_per_pair"] /
                                              arms["fused"]["us_per_pair"], 2),
                     "score_matrix_mib": round(nA * p.B.shape[0] * 4 / 2**20, 1),
                     "identical": lists["fused"] == lists["unfused"]}
    line = {
        "metric": "fused matcher against the unfused arm: us per pair and workspace",
        "value": res["pair_8192x8192"]["speedup"], "unit": "x (unfused / fused time)",
        "higher_is_better": True, "n_gpus": 1, "reps": reps, "data": "synthetic",
        "config": {"workloads": list(res)}, "arms": res,
        "timing": "wall clock over back-to-back calls on one stream after the device warm-up",
    }
    print(json.dumps(line), flush=True)
    return 0 if all(r["identical"] for r in res.values()) else 1


def clock_ramp(serac, synth, torch, np) -> int:
    """How the shader clock and the step time of the 8192 x 8192 benchmark
    grow with back-to-back steps from a cold start: at each checkpoint, 20
    steps timed by wall clock, then the clock the int8 MFMA probe's waves
    see (libserac_probe.so, a ~15 us launch)."""
    p = synth.workload("pair_8192x8192")
    a = torch.from_numpy(p.A).to("cuda:0")
    b = torch.from_numpy(p.B).to("cuda:0")
    out = torch.empty((8192, 2), dtype=torch.int32, device="cuda:0")
    cnt = torch.empty(1, dtype=torch.int32, device="cuda:0")
    prm = p.params()
    torch.cuda.synchronize()
    done, pts = 0, []
    for cp in (0, 5, 25, 100, 300, 1000, 2000, 4000, 7000):
        for _ in range(cp - done):
            serac.match_pair_into(a, b, out, cnt, **prm)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(20):
            serac.match_pair_into(a, b, out, cnt, **prm)
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) / 20 * 1e6
        _, _, ghz = serac.probe_mfma(256, 300, 0)
        done = cp + 20
        pts.append({"steps_before": cp, "us_per_step": round(us, 2), "shader_ghz": round(ghz, 3)})
    line = {"metric": "shader clock and 8192 x 8192 step time against back-to-back steps",
            "value": pts[-1]["shader_ghz"], "unit": "GHz after 7000 steps",
            "higher_is_better": True, "n_gpus": 1, "data": "synthetic", "ramp": pts}
    print(json.dumps(line), flush=True)
    return 0


def f1_probe(serac, synth, torch, np, reps: int = 7) -> int:
    """What cross-pair reuse of A tiles in a batch could save at most.

    A batch workgroup sweeps one 256-row block of A against one pair's B
    (all of it: the exhaustive batch's pairs have one column group).  Its
    time is a fixed part (loading its rows of A, the lane merge, the slot
    and column-best writes) plus one part per 256-column chunk of B.  Reuse
    of the A tile across several B images could remove at most the fixed
    part of every sweep after the first.  Batches of 64 pairs (8 images of
    8192 rows against 8 of nB rows: 2048 workgroups, 8 rounds of 256) with
    nB = 256 c for c = 1 ... 32 chunks give the tile kernel's time per
    round; a least-squares line through them splits it into the fixed part
    and the per-chunk part."""
    warm_device(serac, synth, torch)
    rng = np.random.default_rng(11)
    A = [torch.from_numpy(synth.desc(rng, 8192)).to("cuda:0") for _ in range(8)]
    rows = {}
    rounds = None
    for c in (1, 2, 4, 8, 16, 32):
        B = [torch.from_numpy(synth.desc(rng, 256 * c)).to("cuda:0") for _ in range(8)]
        imgs = A + B
        pairs = [(a, 8 + b) for a in range(8) for b in range(8)]
        serac.match_pairs(imgs, pairs)            # warm-up: workspace, staging
        torch.cuda.synchronize()
        per = []
        for _ in range(reps):
            serac.profile_start(1, 1)
            serac.match_pairs(imgs, pairs)
            torch.cuda.synchronize()
            _, n, ms, name = serac.profile_stop()
            per.append(ms[0] * 1e3)
        units = 64 * 32                            # pairs x row blocks, one column group each
        rounds = -(-units // 256)
        rows[c] = {"kernel": name, "kernel_us_median": round(float(np.median(per)), 3),
                   "us_per_round": round(float(np.median(per)) / rounds, 4)}
    cs = np.array(sorted(rows), dtype=float)
    ts = np.array([rows[int(c)]["us_per_round"] for c in cs])
    slope, fixed = np.polyfit(cs, ts, 1)
    line = {
        "metric": "upper bound on cross-pair A-tile reuse gain, exhaustive batch of 8192-row images",
        "value": round(float(fixed / (fixed + 32 * slope)), 4), "unit": "fraction of tile time",
        "higher_is_better": False, "n_gpus": 1, "reps": reps,
        "fixed_us_per_workgroup": round(float(fixed), 4),
        "chunk_us_per_workgroup": round(float(slope), 4),
        "rounds_per_launch": rounds,
        "per_chunk_count": {str(k): v for k, v in rows.items()},
        "note": "fixed = A-tile load + lane merge + slot/column writes per workgroup; reuse "
                "could save at most the A-tile part of it",
    }
    print(json.dumps(line), flush=True)
    return 0


# Exhaustive image sets (images, descriptors per image) for --strips, and the
# settings compared: the library's test hook SERAC_TEST_STRIP_PAIRS (read at
# the device's set-up, hence one child process per setting) forces pairs
# one by one (1) or strips of up to 16 pairs; unset, the library chooses.
STRIP_SETS = [(200, 512), (128, 1024), (96, 2048), (64, 4096), (48, 8192), (40, 10400)]
STRIP_SETTINGS = [("per_pair", "1"), ("strips_16", "16"), ("library", None)]


def strips_child(serac, synth, torch, np, reps: int) -> int:
    """One setting: tile-kernel time (HIP events on its dispatch) and call
    time per pair for each image set, and a digest of all its lists."""
    out = {}
    for ni, nd in STRIP_SETS:
        bt = synth.image_set(ni, nd, 0.15, 3, 0)
        imgs = [torch.from_numpy(x).to("cuda:0") for x in bt.images]
        bp = bt.pairs.tolist()
        res = serac.match_pairs(imgs, bp)          # warm-up: workspace, staging
        torch.cuda.synchronize()
        tile, wall = [], []
        for _ in range(reps):
            serac.profile_start(1, 1)
            t0 = time.perf_counter()
            res = serac.match_pairs(imgs, bp)
            torch.cuda.synchronize()
            wall.append(time.perf_counter() - t0)
            _, n, ms, name = serac.profile_stop()
            tile.append(ms[0] * 1e3)
        h = hashlib.sha256()
        for r in res:
            h.update(r.cpu().numpy().astype(np.uint32).tobytes())
        out[f"{ni}x{nd}"] = {"pairs": len(bp), "tile_kernel": name,
                             "tile_us_median": round(float(np.median(tile)), 3),
                             "call_us_per_pair_median": round(float(np.median(wall)) * 1e6 / len(bp), 3),
                             "lists_sha256": h.hexdigest()}
    print(json.dumps(out), flush=True)
    return 0


def strips_compare(reps: int = 7) -> int:
    """Cross-pair reuse of A in a batch (strips, serac_tiles_strip) against
    the per-pair sweep (serac_tiles_many) on exhaustive image sets of 512 to
    10400 descriptors per image, each setting in a child process; the lists
    must be identical under every setting."""
    runs = {}
    for label, m in STRIP_SETTINGS:
        env = {k: v for k, v in os.environ.items() if k != "SERAC_TEST_STRIP_PAIRS"}
        if m is not None:
            env["SERAC_TEST_STRIP_PAIRS"] = m
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--strips-child", str(reps)],
                           env=env, capture_output=True, text=True, timeout=900)
        if r.returncode != 0:
            print(r.stderr[-3000:], file=sys.stderr)
            return 1
        runs[label] = json.loads(r.stdout.strip().splitlines()[-1])
        print(f"[strips] {label} done", file=sys.stderr, flush=True)
    sets = {}
    same = True
    for ni, nd in STRIP_SETS:
        key = f"{ni}x{nd}"
        row = {label: runs[label][key] for label, _ in STRIP_SETTINGS}
        digests = {v["lists_sha256"] for v in row.values()}
        same = same and len(digests) == 1
        base = row["per_pair"]["tile_us_median"]
        sets[key] = {
            "pairs": row["per_pair"]["pairs"],
            "chunks_per_pair": -(-nd // 256),
            "tile_us": {label: v["tile_us_median"] for label, v in row.items()},
            "strips_16_vs_per_pair": round(row["strips_16"]["tile_us_median"] / base - 1.0, 4),
            "library_kernel": row["library"]["tile_kernel"],
            "call_us_per_pair": {label: v["call_us_per_pair_median"] for label, v in row.items()},
            "identical_lists": len(digests) == 1,
        }
    line = {"metric": "tile-kernel time of exhaustive image sets, strips of pairs sharing A vs "
                      "pairs one by one", "unit": "us per call (median)", "reps": reps,
            "n_gpus": 1, "sets": sets, "identical_lists": same}
    print(json.dumps(line), flush=True)
    return 0 if same else 1


if __name__ == "__main__":
    sys.exit(main())
