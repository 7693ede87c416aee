"""bench.py's host-side pieces on the CPU: the device-code hash that keys the
committed traffic record, the traffic arithmetic from rocprofv3 counter
CSVs, and the refusal of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_kernel_sha_is_the_device_code():
    h = bench.kernel_sha()
    assert len(h) == 64 and int(h, 16) >= 0
    assert bench.kernel_sha() == h


def _counters(folder, rows):
    os.makedirs(folder)
    with open(os.path.join(folder, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_write_traffic_arithmetic(tmp_path, monkeypatch):
    """Per-dispatch means of the named kernel, scaled by what the counters
    read for the copy probe against its known bytes."""
    k = "void (anonymous namespace)::serac_tiles_fused<true, true>(args)"
    other = "some_other_kernel"
    _counters(tmp_path / "fetch", [(k, "FETCH_SIZE", 1000.0), (k, "FETCH_SIZE", 3000.0),
                                   (other, "FETCH_SIZE", 9e9)])
    _counters(tmp_path / "write", [(k, "WRITE_SIZE", 500.0), (k, "WRITE_SIZE", 700.0)])
    copy = bench.COPY_PROBE_MIB << 20
    # the copy kernel's counters read half the copied bytes (fetch) and all
    # of them (write); a small copy among them is ignored (largest 10 kept)
    cf = [("__amd_rocclr_copyBuffer", "FETCH_SIZE", copy / 2 / 1024)] * 10 + \
         [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 1.0)]
    cw = [("__amd_rocclr_copyBuffer", "WRITE_SIZE", copy / 1024)] * 10
    _counters(tmp_path / "copy_fetch", cf)
    _counters(tmp_path / "copy_write", cw)
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC", str(out))
    assert bench.write_traffic(str(tmp_path), "serac_tiles_fused<true, true>",
                               "pair_8192x8192") == 0
    rec = json.loads(out.read_text())
    assert rec["fetch_size_kib_per_launch"] == 2000.0
    assert rec["write_size_kib_per_launch"] == 600.0
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["bytes_per_launch"] == 2000 * 1024 * 2 + 600 * 1024
    assert rec["dispatches"] == [2, 2]
    assert rec["kernel_sha256"] == bench.kernel_sha()
    # and the bench reads it back as long as the device code matches
    assert bench.measured_traffic()[0] == rec["bytes_per_launch"]
    rec["kernel_sha256"] = "0" * 64
    out.write_text(json.dumps(rec))
    assert bench.measured_traffic()[0] is None


@pytest.mark.parametrize("argv", [["--gpus", "2"], ["--gpus", "8"]])
def test_more_than_one_gpu_is_refused(argv):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
