"""Host-side logic of bench.py (no GPU): the HBM-traffic summary it builds from
rocprofv3 counter CSVs, and its refusal of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

KERNEL = "void gqa::" + bench.HEADLINE_KERNEL + "(gqa::FwdArgs)"
COPY = "__amd_rocclr_copyBuffer"


def _write_counters(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_write_traffic_scales_by_the_calibration_copy(tmp_path):
    fetch, write, out = tmp_path / "fetch.csv", tmp_path / "write.csv", tmp_path / "traffic.json"
    # FETCH_SIZE reads half the bytes of the 256 MiB copy (scale 2); the small
    # copy and the other kernel are ignored; the kernel's dispatches average
    _write_counters(fetch, "FETCH_SIZE", [(COPY, 10.0), (KERNEL, 70000.0), ("void other()", 5.0),
                                         (KERNEL, 72000.0), (COPY, 131072.0)])
    _write_counters(write, "WRITE_SIZE", [(COPY, 262144.0), (KERNEL, 66560.0), (KERNEL, 66560.0)])
    d = bench.write_traffic(str(fetch), str(write), 256, out_path=str(out))
    assert d["fetch_scale"] == pytest.approx(2.0) and d["write_scale"] == pytest.approx(1.0)
    assert d["read_bytes_per_launch"] == pytest.approx(71000.0 * 2.0 * 1024)
    assert d["write_bytes_per_launch"] == pytest.approx(66560.0 * 1024)
    assert d["hbm_bytes_per_launch"] == pytest.approx(d["read_bytes_per_launch"] + d["write_bytes_per_launch"])
    assert d["kernel"] == KERNEL
    assert d["kernel_digest"] == bench.kernel_digest(bench.FWD_SOURCES)
    assert json.loads(out.read_text()) == d


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
