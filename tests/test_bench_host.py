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


def test_write_counters_busy_fraction_and_clock(tmp_path):
    """Per dispatch: mfma_busy = (busy / 1024 SIMDs) / (GRBM_GUI_ACTIVE / 8
    XCDs), clock = (GRBM_GUI_ACTIVE / 8) / duration; dispatches average and
    other kernels are kept apart."""
    path, out = tmp_path / "sq.csv", tmp_path / "counters.json"
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    other = "void gqa::attn_bwd_dkv2_kernel<128, true>(gqa::BwdArgs, int)"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        # dispatch 1: 800000 cycles per XCD over 400 us -> 2.0 GHz; busy 0.5 of them on every SIMD
        for name, val in (("GRBM_GUI_ACTIVE", 8 * 800000.0), ("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 400000.0)):
            w.writerow({"Dispatch_Id": 1, "Kernel_Name": KERNEL, "Counter_Name": name, "Counter_Value": val,
                        "Start_Timestamp": 1000, "End_Timestamp": 1000 + 400000})
        # dispatch 2: 1.5 GHz, busy 0.7
        for name, val in (("GRBM_GUI_ACTIVE", 8 * 600000.0), ("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 420000.0)):
            w.writerow({"Dispatch_Id": 2, "Kernel_Name": KERNEL, "Counter_Name": name, "Counter_Value": val,
                        "Start_Timestamp": 5000000, "End_Timestamp": 5000000 + 400000})
        for name, val in (("GRBM_GUI_ACTIVE", 8 * 100.0), ("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 10.0)):
            w.writerow({"Dispatch_Id": 3, "Kernel_Name": other, "Counter_Name": name, "Counter_Value": val,
                        "Start_Timestamp": 0, "End_Timestamp": 100})
        w.writerow({"Dispatch_Id": 4, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "GRBM_GUI_ACTIVE",
                    "Counter_Value": 5.0, "Start_Timestamp": 0, "End_Timestamp": 10})
    d = bench.write_counters(str(path), "causal_b1_k8_g4_t8192_h128", out_path=str(out))
    k = d["kernels"][KERNEL]
    assert k["dispatches"] == 2
    assert k["clock_ghz"] == pytest.approx(700000.0 / 400000.0)
    assert k["mfma_busy"] == pytest.approx(410000.0 / 700000.0)
    assert k["duration_us"] == pytest.approx(400.0)
    assert d["kernels"][other]["mfma_busy"] == pytest.approx(0.1)
    assert "__amd_rocclr_copyBuffer" not in d["kernels"]
    assert d["source_digest"] == bench.kernel_digest(bench.ALL_SOURCES)
    assert json.loads(out.read_text()) == d


def test_counter_figures_need_matching_sources(tmp_path, monkeypatch):
    roof = {"frac": 0.5, "traffic": 2e8, "algorithmic_hbm_bytes_per_launch": 1.6e8}
    monkeypatch.setattr(bench, "counters_file", lambda w: str(tmp_path / "c.json"))
    (tmp_path / "c.json").write_text(json.dumps({"source_digest": "stale", "kernels": {
        KERNEL: {"mfma_busy": 0.7, "clock_ghz": 2.0, "duration_us": 440.0}}}))
    bench.add_counter_figures(roof, "w", bench.HEADLINE_KERNEL, 0.4)
    assert roof["mfma_busy"] is None and roof["clock_ghz"] is None and roof["frac_at_clock"] is None
    assert roof["hbm_gbps"] == pytest.approx(2e8 / 0.4e-3 / 1e9)
    (tmp_path / "c.json").write_text(json.dumps({"source_digest": bench.kernel_digest(bench.ALL_SOURCES), "kernels": {
        KERNEL: {"mfma_busy": 0.7, "clock_ghz": 2.0, "duration_us": 440.0}}}))
    bench.add_counter_figures(roof, "w", bench.HEADLINE_KERNEL, 0.4)
    assert roof["mfma_busy"] == 0.7 and roof["frac_at_clock"] == pytest.approx(0.5 * 2.4 / 2.0)


def test_finish_exits_3_on_a_parity_miss(capsys):
    bench.finish({"value": 1.0, "cpu_baseline": {"parity_ok": True}})
    assert json.loads(capsys.readouterr().out)["value"] == 1.0
    with pytest.raises(SystemExit) as e:
        bench.finish({"value": 1.0, "cpu_baseline": {"parity_ok": False}})
    assert e.value.code == 3


def test_pair_counts_match_a_brute_force_mask():
    """The visible-pair counts behind the window and prefill FLOP figures,
    against counting a dense boolean mask."""
    import numpy as np
    from workloads import end_aligned_pairs, window_pairs
    for T, S in [(1, 1), (5, 9), (9, 5), (16, 16), (7, 40)]:
        t, s = np.arange(T)[:, None], np.arange(S)[None, :]
        assert end_aligned_pairs(T, S) == int((s <= t + S - T).sum()), (T, S)
        for wl in (0, 3, 100):
            band = (s <= t) & (s >= t - wl)
            assert window_pairs(T, S, wl) == int(band.sum()), (T, S, wl)
