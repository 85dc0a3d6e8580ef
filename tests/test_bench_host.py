"""Host logic of bench.py that needs no GPU: which kernel the roofline object
names, the HBM traffic record (counter means over a rocprofv3 CSV, scaling by
the calibration copy, the lookup that drops a record once the kernel's
sources change), and the refusal of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_roofline_kernel_by_path():
    assert bench.roofline_kernel(64, False)[0] == "skinny_kernel<0, false>"
    assert bench.roofline_kernel(64, True)[0] == "skinny_kernel<0, true>"
    assert bench.roofline_kernel(65, False)[0] == "gemm_kernel<0, true>"
    assert bench.roofline_kernel(16384, True)[0] == "gemm_fp8_kernel<0>"
    for n, f in ((64, False), (16384, True)):
        for path in bench.roofline_kernel(n, f)[1]:
            assert os.path.exists(path)
    assert bench.traffic_key("prefill", True) == "prefill_fp8"


def _write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, grid, value) in enumerate(rows):
            w.writerow([i, grid, name, counter, value])


def test_traffic_record_roundtrip(tmp_path, monkeypatch):
    # the routed launches (large grid) and a shared-expert launch of the same
    # kernel (small grid), and a 1 GiB copy that reads as 2^19 KiB fetched
    kern = "void moe::gemm_fp8_kernel<0>(moe::GemmArgs)"
    fetch = [(kern, 4096, 1000.0), (kern, 4096, 1200.0), (kern, 512, 50.0),
             ("__amd_rocclr_copyBuffer", 131072, 524288.0), ("__amd_rocclr_copyBuffer", 512, 3.0)]
    write = [(kern, 4096, 100.0), (kern, 4096, 100.0), (kern, 512, 5.0),
             ("__amd_rocclr_copyBuffer", 131072, 1048576.0)]
    fd, wd = str(tmp_path / "f"), str(tmp_path / "w")
    _write_counters(fd, "FETCH_SIZE", fetch)
    _write_counters(wd, "WRITE_SIZE", write)
    mean, cp, n = bench._counter_means(fd, "FETCH_SIZE", "gemm_fp8_kernel<0>")
    assert (mean, cp, n) == (1100.0, 524288.0, 2)
    tf = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tf))
    bench.record_traffic("prefill", 16384, True, fd, wd, 1024)
    rec = json.load(open(tf))["prefill_fp8"]
    assert rec["kernel_name"] == "gemm_fp8_kernel<0>"
    assert rec["fetch_bytes_per_launch"] == pytest.approx(1100.0 * 2 * 1024)
    assert rec["write_bytes_per_launch"] == pytest.approx(100.0 * 1024)
    assert bench.traffic_for("prefill", 16384, True) == pytest.approx(rec["bytes_per_launch"])
    # another path, another record; a changed source hash drops it
    assert bench.traffic_for("prefill", 16384, False) is None
    rec["source_sha256_16"] = "0" * 16
    json.dump({"prefill_fp8": rec}, open(tf, "w"))
    assert bench.traffic_for("prefill", 16384, True) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
