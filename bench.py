#!/usr/bin/env python3
"""Benchmark of the fused GQA flash-attention forward on one MI355X.

Workload: causal grouped-query attention forward, B=1, K=8 kv heads, G=4
(32 query heads), T=S=8192, H=128, bf16 inputs ~ N(0,1) (q pre-scaled by
H^-1/2), synthetic and seeded. One step = one attn_fwd call over the whole
batch; inputs are resident in HBM before the timed region. Before the W
warm-up steps, about one second of the same launches lets the GPU clock settle
(untimed).

Prints ONE JSON line. `value` is forward TFLOP/s with causal FLOPs counted
as the executed half, 4*B*K*G*T*S*H/2. `roofline` compares the forward
kernel's average launch time (HIP events on the launch stream) with the
MI355X dense bf16 MFMA peak; `cpu_baseline` times the CPU oracle on a
bounded random sample of the same workload's query rows on the host cores.
A second leg times the backward (dQ, dK, dV from the saved lse) on the same
tensors and reports it under "backward".

--workload window times the headline shape with a causal sliding window of
1024 keys (attn_fwd_local, attn_bwd_local), FLOPs counted on visible pairs.

--workload long times the 32k-token shape B=1, K=2, G=8, T=S=32768, H=256
(causal) in the same format, without the backward leg.

--workload segments times the packed-sequence shape B=4, K=8, G=4, T=S=2048,
H=128 (causal and segment ids, segments of 64-1024 tokens) in the same
format; value and the roofline fraction count only the visible (t, s) pairs
(the work the kernel executes), with the causal-half rate beside them. Its
backward leg, with the same segment ids, counts the visible pairs too.

--workload prefill times a chunk of T=1024 new queries at the end of an
S=8192 context (B=1, K=8, G=4, H=128, end-aligned causal) through the tuned
split-KV forward, FLOPs counted on visible pairs, with the single pass beside it.

--write-traffic FETCH_CSV WRITE_CSV turns two rocprofv3 --pmc runs (FETCH_SIZE,
then WRITE_SIZE, each with --copy-calibration-mib) into the HBM bytes per
launch of the headline forward kernel, scaled by what the same counters read
for the calibration copy, and stores them with a digest of the kernel source.

--write-counters SQ_CSV turns a rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES
GRBM_GUI_ACTIVE run of a workload into each kernel's MFMA-busy fraction and
running clock (GRBM_GUI_ACTIVE per XCD over the dispatch's own duration), stored
with a digest of the kernel sources; the bench line reports them, and the
fraction of the peak at that clock, while the digest matches.

The CPU baseline times the float-accumulation build of the oracle source on a
sample of the workload's rows (the fp64 build's rate beside it), and checks
the GPU output against the fp64 oracle on its own sample: a miss of max-abs
2e-2 or rel-L2 5e-3 marks the line "parity_ok": false and exits with status 3.

--workload decode instead times the decoding shape B=16, K=8, G=4, T=1,
S=32768, H=128 (non-causal: the query sees the whole context) through the
split-KV forward (attn_fwd_ws), and prints one JSON line whose value is the
HBM bandwidth achieved on the algorithmic bytes (q, k, v, o, lse once each),
with the single-pass forward's time beside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MI355X_BF16_DENSE_TFLOPS = 2500.0   # published dense bf16 MFMA peak
MI355X_HBM_GBPS = 8000.0            # published HBM3E bandwidth
MI355X_PEAK_CLOCK_GHZ = 2.4         # the engine clock the published peak assumes
MI355X_XCDS = 8
MI355X_SIMDS = 1024                 # 256 CUs x 4
O_MAX_ABS, O_REL_L2 = 2e-2, 5e-3    # parity bar of the sampled check
METRIC = "attention TFLOP/s (fwd, causal) at 1 GPU; % of bf16 MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_causal_b1_k8_g4_t8192_h128_traffic.json")
FWD_SOURCES = ["grouped_query_attention_flash_amd/csrc/attn_fwd.hip",
               "grouped_query_attention_flash_amd/csrc/gqa_device.h"]
ALL_SOURCES = FWD_SOURCES + ["grouped_query_attention_flash_amd/csrc/attn_bwd.hip",
                             "grouped_query_attention_flash_amd/csrc/gqa_launch.h",
                             "grouped_query_attention_flash_amd/csrc/api.hip"]


def counters_file(workload):
    return os.path.join(ROOT, "profiles", "%s_counters.json" % workload)


def write_counters(sq_csv, workload, out_path=None):
    """Per-kernel MFMA-busy fraction and running clock from one rocprofv3 --pmc
    SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE run (its counter CSV carries each
    dispatch's start and end time). SQ_VALU_MFMA_BUSY_CYCLES sums over the
    chip's SIMDs and GRBM_GUI_ACTIVE over its XCDs, so per dispatch
      mfma_busy = (busy / 1024 SIMDs) / (GRBM_GUI_ACTIVE / 8 XCDs)
      clock     = (GRBM_GUI_ACTIVE / 8 XCDs) / duration."""
    import csv
    disp = {}
    with open(sq_csv) as f:
        for r in csv.DictReader(f):
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            d = disp.setdefault(key, {"dur_ns": float(r["End_Timestamp"]) - float(r["Start_Timestamp"])})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
    kernels = {}
    for (_, name), d in disp.items():
        if "SQ_VALU_MFMA_BUSY_CYCLES" not in d or "GRBM_GUI_ACTIVE" not in d or d["dur_ns"] <= 0:
            continue
        if "gqa::" not in name:
            continue
        k = kernels.setdefault(name, {"dispatches": 0, "busy": 0.0, "grbm": 0.0, "dur_ns": 0.0})
        k["dispatches"] += 1
        k["busy"] += d["SQ_VALU_MFMA_BUSY_CYCLES"]
        k["grbm"] += d["GRBM_GUI_ACTIVE"]
        k["dur_ns"] += d["dur_ns"]
    out = {}
    for name, k in kernels.items():
        n = k["dispatches"]
        cyc = k["grbm"] / n / MI355X_XCDS
        out[name] = {"dispatches": n, "duration_us": k["dur_ns"] / n / 1e3,
                     "mfma_busy": (k["busy"] / n / MI355X_SIMDS) / cyc,
                     "clock_ghz": cyc / (k["dur_ns"] / n)}
    d = {"workload": workload, "source_digest": kernel_digest(ALL_SOURCES),
         "counters": "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE", "kernels": out}
    path = out_path or counters_file(workload)
    with open(path, "w") as f:
        json.dump(d, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(d))
    return d


def measured_counters(workload, kernel_substr):
    """(mfma_busy, clock_ghz) of the kernel whose name contains kernel_substr,
    from the committed counter file of the workload, or None if missing or
    taken on other kernel sources."""
    try:
        with open(counters_file(workload)) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_digest") != kernel_digest(ALL_SOURCES):
        return None
    for name, k in d.get("kernels", {}).items():
        if kernel_substr in name:
            return k
    return None


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def kernel_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from committed rocprofv3 counter runs, or None if
    missing or taken on a different version of the kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_digest") != kernel_digest(FWD_SOURCES):
        return None
    return d.get("hbm_bytes_per_launch")


HEADLINE_KERNEL = "attn_fwd_pp_kernel<128, 64, true, false, false, 0, true>"


def write_traffic(fetch_csv, write_csv, calib_mib, out_path=TRAFFIC_FILE):
    """HBM bytes per launch of the headline forward kernel from two rocprofv3
    --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch). Each counter
    is scaled by bytes / reading of the largest device copy in the same run
    (the calibration copy of calib_mib MiB, which reads and writes that much)."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    calib = calib_mib * 1024.0  # KiB moved each way by the copy
    fetch_copy = max(v for k, vs in fetch.items() if "copyBuffer" in k for v in vs)
    write_copy = max(v for k, vs in write.items() if "copyBuffer" in k for v in vs)
    fetch_scale, write_scale = calib / fetch_copy, calib / write_copy
    name = next(k for k in fetch if HEADLINE_KERNEL in k)
    rd = sum(fetch[name]) / len(fetch[name]) * fetch_scale * 1024.0
    wr = sum(write[name]) / len(write[name]) * write_scale * 1024.0
    d = {"kernel": name, "kernel_digest": kernel_digest(FWD_SOURCES), "workload": "causal_b1_k8_g4_t8192_h128",
         "fetch_scale": fetch_scale, "write_scale": write_scale, "read_bytes_per_launch": rd,
         "write_bytes_per_launch": wr, "hbm_bytes_per_launch": rd + wr}
    with open(out_path, "w") as f:
        json.dump(d, f, indent=1)
        f.write("\n")
    print(json.dumps(d))
    return d


def settle_clock(fn, seconds=1.0):
    """Run launches for about `seconds` before the warm-up steps: the GPU's
    clock ramps up over the first tens of milliseconds of sustained load, and a
    timed region that starts before that measures the ramp, not the kernel."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()


def time_launches(fn, steps, warmup, settle_s=1.0):
    import torch
    if settle_s > 0:
        settle_clock(fn, settle_s)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps  # ms per launch


def _sample_rows(total_rows, per_row_s, target_s, rng, n0):
    n = int(min(total_rows, max(n0, target_s / max(per_row_s, 1e-9))))
    return np.sort(rng.choice(total_rows, size=n, replace=False)) if n < total_rows else np.arange(total_rows)


def cpu_baseline(inp, w, o_gpu, target_s=8.0, row_flops=None, oracle_kw=None, total_flops=None):
    """The oracle on the host cores, on bounded samples of the workload's query
    rows: the float-accumulation build of the oracle source is timed (value),
    the fp64 build both timed (fp64_value) and compared with the GPU output on
    its rows (parity_ok: max-abs <= 2e-2 and rel-L2 <= 5e-3)."""
    import oracle
    from workloads import attention_flops

    oracle_kw = dict(oracle_kw or {"causal": w.causal})
    threads = oracle.max_threads()
    rng = np.random.default_rng(12345)
    total_rows = w.B * w.K * w.G * w.T
    if row_flops is None:
        def row_flops(rows):
            t = rows % w.T
            visible = (t + 1) if w.causal else np.full_like(t, w.S)
            return float(4.0 * w.H * visible.sum())
    full = total_flops or attention_flops(w.B, w.K, w.G, w.T, w.S, w.H, w.causal)
    legs = {}
    for prec in ("f64", "f32"):
        n0 = min(2048, total_rows)
        rows = np.sort(rng.choice(total_rows, size=n0, replace=False))
        t0 = time.perf_counter()
        oracle.fwd(inp["q"], inp["k"], inp["v"], rows=rows, precision=prec, **oracle_kw)
        per_row = (time.perf_counter() - t0) / n0
        rows = _sample_rows(total_rows, per_row, target_s, rng, n0)
        t0 = time.perf_counter()
        ref_o, _ = oracle.fwd(inp["q"], inp["k"], inp["v"], rows=rows, precision=prec, **oracle_kw)
        elapsed = time.perf_counter() - t0
        legs[prec] = (rows, ref_o, elapsed, row_flops(rows))
    rows, ref_o, elapsed64, flops64 = legs["f64"]
    got = o_gpu.reshape(-1, w.H)[torch_index(rows, o_gpu.device)].float().cpu().numpy()
    err = float(np.abs(got - ref_o).max())
    rel = float(np.linalg.norm(got - ref_o) / np.linalg.norm(ref_o))
    rows32, _, elapsed32, flops32 = legs["f32"]
    return {
        "value": flops32 / elapsed32 / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "cpu_model": host_cpu_model(),
        "sample": "%d random query rows (%.3g of the workload's FLOPs) through the float-accumulation build of "
                  "the oracle source, %.1f s; the fp64 build on %d rows (%.3g), %.1f s" % (
                      len(rows32), flops32 / full, elapsed32, len(rows), flops64 / full, elapsed64),
        "fp64_value": flops64 / elapsed64 / 1e12,
        "sample_max_abs_vs_gpu": err,
        "sample_rel_l2_vs_gpu": rel,
        "parity_ok": bool(err <= O_MAX_ABS and rel <= O_REL_L2),
        "rows": int(len(rows32)),
        "elapsed_s": elapsed32,
    }


def torch_index(rows, device):
    import torch
    return torch.from_numpy(np.asarray(rows, dtype=np.int64)).to(device)


def decode_bench(args):
    """The decoding workload through the split-KV forward: HBM-bound."""
    import torch
    import grouped_query_attention_flash_amd as gqa
    from workloads import DECODE, attention_flops, make_qkv

    w = DECODE
    q, k, v = make_qkv(w.B, w.K, w.G, w.T, w.S, w.H, w.seed)
    inp_cpu = {"q": q, "k": k, "v": v}
    dev = torch.device("cuda", 0)
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty(w.B, w.K, w.G, w.T, dtype=torch.float32, device=dev)
    n_splits = gqa.attn_fwd_split_count(w.B, w.K, w.G, w.T, w.S, w.H)
    ws = torch.empty(max(1, gqa.attn_fwd_workspace_bytes(w.B, w.K, w.G, w.T, w.S, w.H)), dtype=torch.uint8,
                     device=dev)
    torch.cuda.synchronize()

    def step():
        gqa.attn_fwd(qd, kd, vd, causal=w.causal, out=o, lse=lse, split_kv=True, workspace=ws)

    def step_single():
        gqa.attn_fwd(qd, kd, vd, causal=w.causal, out=o, lse=lse)

    ms_single = time_launches(step_single, max(5, args.steps // 2), max(2, args.warmup // 2), args.settle_seconds)
    ms = time_launches(step, args.steps, args.warmup, args.settle_seconds)
    hbm_bytes = 2 * (qd.numel() + kd.numel() + vd.numel() + o.numel()) + 4 * lse.numel()
    gbps = hbm_bytes / (ms * 1e-3) / 1e9
    flops = attention_flops(w.B, w.K, w.G, w.T, w.S, w.H, w.causal)
    result = {
        "metric": "decode attention HBM GB/s (fwd, T=1, split-KV) at 1 GPU; % of HBM peak",
        "value": gbps,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, q pre-scaled by H^-1/2)",
        "config": {"workload": w.name, "B": w.B, "K": w.K, "G": w.G, "T": w.T, "S": w.S, "H": w.H,
                   "causal": w.causal, "n_splits": n_splits},
        "roofline": {
            "kernel": "attn_fwd_decode_kernel<128,4> split-KV + attn_fwd_merge_kernel (whole call)",
            "bound": "hbm",
            "achieved": gbps,
            "peak": MI355X_HBM_GBPS,
            "unit": "GB/s",
            "frac": gbps / MI355X_HBM_GBPS,
            "traffic": None,
            "algorithmic_hbm_bytes_per_launch": hbm_bytes,
            "algorithmic_flops_per_launch": flops,
        },
        "single_pass": {"ms": ms_single, "gbps": hbm_bytes / (ms_single * 1e-3) / 1e9},
    }
    if not args.no_cpu_baseline:
        step()
        torch.cuda.synchronize()
        cb = cpu_baseline(inp_cpu, w, o)
        # the oracle's rate in the metric's unit: each sampled row stands for
        # its share of the launch's algorithmic bytes
        total_rows = w.B * w.K * w.G * w.T
        to_gbps = (hbm_bytes / flops) * 1e3  # TFLOP/s -> GB/s at the launch's bytes per FLOP
        cb["value_tflops"], cb["fp64_value_tflops"] = cb["value"], cb["fp64_value"]
        cb["value"] = cb["rows"] / total_rows * hbm_bytes / cb["elapsed_s"] / 1e9
        cb["fp64_value"] = cb["fp64_value"] * to_gbps
        cb["unit"] = "GB/s"
        result["cpu_baseline"] = cb
    finish(result)


def window_bench(args):
    """The headline shape with a causal sliding window (attn_fwd_local /
    attn_bwd_local): MFMA-bound, FLOPs counted on the visible pairs."""
    import torch
    import grouped_query_attention_flash_amd as gqa
    from workloads import WINDOW, WINDOW_LEFT, make_qkv, window_pairs

    w = WINDOW
    win = (WINDOW_LEFT, -1)
    q, k, v, do = make_qkv(w.B, w.K, w.G, w.T, w.S, w.H, w.seed, with_do=True)
    dev = torch.device("cuda", 0)
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    o = torch.empty_like(qd)
    lse = torch.empty(w.B, w.K, w.G, w.T, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step():
        gqa.attn_fwd(qd, kd, vd, causal=True, out=o, lse=lse, window=win)

    ms = time_launches(step, args.steps, args.warmup, args.settle_seconds)
    pairs = window_pairs(w.T, w.S, WINDOW_LEFT) * w.B * w.K * w.G
    flops = 4.0 * w.H * pairs
    tflops = flops / (ms * 1e-3) / 1e12
    result = {
        "metric": "sliding-window attention TFLOP/s (fwd, causal, window 1024) at 1 GPU; % of bf16 MFMA peak",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, q pre-scaled by H^-1/2)",
        "config": {"workload": w.name, "B": w.B, "K": w.K, "G": w.G, "T": w.T, "S": w.S, "H": w.H,
                   "causal": True, "window_left": WINDOW_LEFT, "window_right": -1},
        "roofline": {
            "kernel": "attn_fwd_pp_kernel<128,64,true,true,false,0,true> (ping-pong, windowed, persistent grid)",
            "bound": "mfma",
            "achieved": tflops,
            "peak": MI355X_BF16_DENSE_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / MI355X_BF16_DENSE_TFLOPS,
            "traffic": None,
            "algorithmic_flops_per_launch": flops,
            "visible_pairs": pairs,
        },
    }
    if not args.no_backward:
        ws = torch.empty(gqa.attn_bwd_workspace_bytes(w.B, w.K, w.G, w.T, w.S, w.H), dtype=torch.uint8, device=dev)
        dq = torch.empty(qd.shape, dtype=torch.float32, device=dev)
        dk = torch.empty(kd.shape, dtype=torch.float32, device=dev)
        dv = torch.empty(vd.shape, dtype=torch.float32, device=dev)
        step()

        def bstep():
            gqa.attn_bwd(qd, kd, vd, o, lse, dod, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws, window=win)

        bms = time_launches(bstep, max(5, args.steps // 2), max(2, args.warmup // 2), args.settle_seconds)
        result["backward"] = {"ms": bms, "tflops": 2.5 * flops / (bms * 1e-3) / 1e12,
                              "flops_convention": "2.5x forward (5 matmuls per visible pair)"}
    if not args.no_cpu_baseline:
        step()
        torch.cuda.synchronize()

        def row_flops(rows):
            t = rows % w.T
            return float(4.0 * w.H * (np.minimum(t, w.S - 1) - np.maximum(0, t - win[0]) + 1).sum())

        result["cpu_baseline"] = cpu_baseline({"q": q, "k": k, "v": v}, w, o, row_flops=row_flops,
                                              oracle_kw={"causal": True, "window": win}, total_flops=flops)
    finish(result)


def prefill_bench(args):
    """A chunk of new queries at the end of a cached context (end-aligned
    causal) through the tuned split-KV forward: MFMA-bound, FLOPs counted on
    the visible pairs, the single pass timed beside it."""
    import torch
    import grouped_query_attention_flash_amd as gqa
    from workloads import PREFILL, PREFILL_CAUSAL, end_aligned_pairs, make_qkv

    w = PREFILL
    q, k, v = make_qkv(w.B, w.K, w.G, w.T, w.S, w.H, w.seed)
    dev = torch.device("cuda", 0)
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty(w.B, w.K, w.G, w.T, dtype=torch.float32, device=dev)
    n_splits = gqa.attn_fwd_split_count(w.B, w.K, w.G, w.T, w.S, w.H)
    ws = torch.empty(max(1, gqa.attn_fwd_workspace_bytes(w.B, w.K, w.G, w.T, w.S, w.H)), dtype=torch.uint8,
                     device=dev)
    torch.cuda.synchronize()

    def step():
        gqa.attn_fwd(qd, kd, vd, causal=PREFILL_CAUSAL, out=o, lse=lse, split_kv=True, workspace=ws)

    def step_single():
        gqa.attn_fwd(qd, kd, vd, causal=PREFILL_CAUSAL, out=o, lse=lse)

    ms_single = time_launches(step_single, max(5, args.steps // 2), max(2, args.warmup // 2), args.settle_seconds)
    ms = time_launches(step, args.steps, args.warmup, args.settle_seconds)
    pairs = end_aligned_pairs(w.T, w.S) * w.B * w.K * w.G
    flops = 4.0 * w.H * pairs
    tflops = flops / (ms * 1e-3) / 1e12
    hbm_bytes = 2 * (qd.numel() + kd.numel() + vd.numel() + o.numel()) + 4 * lse.numel()
    result = {
        "metric": "chunked-prefill attention TFLOP/s (fwd, end-aligned causal, T=1024 after 7168 cached keys) "
                  "at 1 GPU; % of bf16 MFMA peak",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, q pre-scaled by H^-1/2)",
        "config": {"workload": w.name, "B": w.B, "K": w.K, "G": w.G, "T": w.T, "S": w.S, "H": w.H,
                   "causal": "end-aligned", "n_splits": n_splits},
        "roofline": {
            "kernel": "attn_fwd_pp_split_kernel<128,64,true,false> + attn_fwd_merge_kernel (whole call)",
            "bound": "mfma",
            "achieved": tflops,
            "peak": MI355X_BF16_DENSE_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / MI355X_BF16_DENSE_TFLOPS,
            "traffic": None,
            "algorithmic_flops_per_launch": flops,
            "algorithmic_hbm_bytes_per_launch": hbm_bytes,
            "visible_pairs": pairs,
        },
        "single_pass": {"ms": ms_single, "tflops": flops / (ms_single * 1e-3) / 1e12},
    }
    if not args.no_cpu_baseline:
        step()
        torch.cuda.synchronize()

        def row_flops(rows):
            t = rows % w.T
            return float(4.0 * w.H * (t + w.S - w.T + 1).sum())

        result["cpu_baseline"] = cpu_baseline({"q": q, "k": k, "v": v}, w, o, row_flops=row_flops,
                                              oracle_kw={"causal": PREFILL_CAUSAL}, total_flops=flops)
    finish(result)


def finish(result):
    """Print the one JSON line; a sampled parity miss exits with status 3."""
    print(json.dumps(result), flush=True)
    cb = result.get("cpu_baseline")
    if cb is not None and not cb.get("parity_ok", True):
        print("parity miss: the GPU output differs from the oracle beyond max-abs %.0e / rel-L2 %.0e "
              "on the sampled rows" % (O_MAX_ABS, O_REL_L2), file=sys.stderr)
        sys.exit(3)


def add_counter_figures(roof, workload, kernel_substr, ms):
    """MFMA-busy fraction, running clock and the fraction of the peak at that
    clock from the committed counter file (None when it was taken on other
    kernel sources), and HBM GB/s from the measured traffic."""
    c = measured_counters(workload, kernel_substr)
    roof["mfma_busy"] = c["mfma_busy"] if c else None
    roof["clock_ghz"] = c["clock_ghz"] if c else None
    roof["frac_at_clock"] = roof["frac"] * MI355X_PEAK_CLOCK_GHZ / c["clock_ghz"] if c else None
    roof["counters_kernel_us"] = c["duration_us"] if c else None
    roof["counters_file"] = os.path.relpath(counters_file(workload), ROOT) if c else None
    alg = roof.get("algorithmic_hbm_bytes_per_launch")
    roof["algorithmic_hbm_gbps"] = alg / (ms * 1e-3) / 1e9 if alg else None
    roof["hbm_gbps"] = roof["traffic"] / (ms * 1e-3) / 1e9 if roof.get("traffic") else None
    roof["hbm_frac"] = roof["hbm_gbps"] / MI355X_HBM_GBPS if roof["hbm_gbps"] else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward leg")
    ap.add_argument("--settle-seconds", type=float, default=1.0,
                    help="untimed launches before the warm-up steps, for the clock to settle")
    ap.add_argument("--workload", choices=["headline", "decode", "window", "prefill", "long", "segments"],
                    default="headline",
                    help="headline: the causal T=S=8192 forward (default); decode: T=1 against S=32768; "
                         "window: the headline shape with a causal 1024-key sliding window; "
                         "prefill: 1024 end-aligned causal queries against S=8192 through the split-KV forward; "
                         "long: the causal T=S=32768 H=256 forward; "
                         "segments: the packed-sequence T=S=2048 forward with segment ids")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the headline kernel's HBM bytes per launch from two rocprofv3 --pmc CSVs "
                         "(needs --copy-calibration-mib, the size those runs copied) and exit")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB three times (a known-size "
                         "reference dispatch for the HBM byte counters)")
    ap.add_argument("--write-counters", metavar="SQ_CSV",
                    help="write the workload's per-kernel MFMA-busy fraction and clock from a rocprofv3 --pmc "
                         "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE counter CSV and exit")
    args = ap.parse_args()
    if args.write_traffic:
        if not args.copy_calibration_mib:
            ap.error("--write-traffic needs --copy-calibration-mib")
        write_traffic(args.write_traffic[0], args.write_traffic[1], args.copy_calibration_mib)
        return
    if args.write_counters:
        from workloads import workload_by_bench_name
        write_counters(args.write_counters, workload_by_bench_name(args.workload).name)
        return
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path (--gpus %d refused)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import grouped_query_attention_flash_amd as gqa
    from workloads import HEADLINE, WORKLOADS, attention_flops, make_qkv, make_segment_ids, visible_pairs_flops

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.workload == "decode":
        decode_bench(args)
        return
    if args.workload == "window":
        window_bench(args)
        return
    if args.workload == "prefill":
        prefill_bench(args)
        return
    w = HEADLINE
    kernel = "attn_fwd_pp_kernel<128,64,true,false,false,0,true> (ping-pong, dense causal, persistent grid)"
    kernel_substr = "attn_fwd_pp_kernel<128, 64, true, false, false, 0, true>"
    seg = None
    if args.workload == "long":
        w = WORKLOADS["causal_b1_k2_g8_t32768_h256"]
        kernel = "attn_fwd_pp_kernel<256,32,true,false,false,0,false> (ping-pong, dense causal)"
        kernel_substr = "attn_fwd_pp_kernel<256, 32, true, false, false, 0, false>"
        args.no_backward = True
    elif args.workload == "segments":
        w = WORKLOADS["segments_causal_b4_k8_g4_t2048_h128"]
        kernel = "attn_fwd_pp_kernel<128,64,true,false,true,2,false> (ping-pong, causal with segment ids; loads spread over the MFMA phase)"
        kernel_substr = "attn_fwd_pp_kernel<128, 64, true, false, true, 2, false>"
        seg = make_segment_ids(w.B, w.T, w.seed)
    t = make_qkv(w.B, w.K, w.G, w.T, w.S, w.H, w.seed, with_do=not args.no_backward)
    q, k, v = t[:3]
    inp_cpu = {"q": q, "k": k, "v": v}
    dev = torch.device("cuda", 0)
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    dod = None if args.no_backward else t[3].to(dev)
    o = torch.empty_like(qd)
    lse = torch.empty(w.B, w.K, w.G, w.T, dtype=torch.float32, device=dev)
    segd = None if seg is None else seg.to(dev)
    torch.cuda.synchronize()

    def step():
        gqa.attn_fwd(qd, kd, vd, causal=w.causal, q_seg=segd, kv_seg=segd, out=o, lse=lse)

    ms = time_launches(step, args.steps, args.warmup, args.settle_seconds)
    flops = attention_flops(w.B, w.K, w.G, w.T, w.S, w.H, w.causal)
    causal_half_flops = flops
    if seg is not None:
        # packed segments: the executed work is the visible pairs only
        flops = visible_pairs_flops(w.H, w.K, w.G, seg, causal=True)
    tflops = flops / (ms * 1e-3) / 1e12
    fwd_bytes = 2 * (qd.numel() + kd.numel() + vd.numel() + o.numel()) + 4 * lse.numel()
    if seg is not None:
        fwd_bytes += 4 * 2 * seg.numel()

    result = {
        "metric": METRIC if seg is None else
        "attention TFLOP/s (fwd, causal, packed segments; visible pairs) at 1 GPU; % of bf16 MFMA peak",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, q pre-scaled by H^-1/2)",
        "config": {"workload": w.name, "B": w.B, "K": w.K, "G": w.G, "T": w.T, "S": w.S, "H": w.H,
                   "causal": w.causal, "mask": "lazy causal" if seg is None else "lazy causal and segment ids"},
        "pct_of_peak": 100.0 * tflops / MI355X_BF16_DENSE_TFLOPS,
        "roofline": {
            "kernel": kernel,
            "bound": "mfma",
            "achieved": tflops,
            "peak": MI355X_BF16_DENSE_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / MI355X_BF16_DENSE_TFLOPS,
            "traffic": measured_traffic() if w is HEADLINE else None,
            "algorithmic_flops_per_launch": flops,
            "algorithmic_hbm_bytes_per_launch": fwd_bytes,
        },
    }

    add_counter_figures(result["roofline"], w.name, kernel_substr, ms)
    if seg is not None:
        result["causal_half"] = {"flops_per_launch": causal_half_flops,
                                 "tflops": causal_half_flops / (ms * 1e-3) / 1e12,
                                 "visible_fraction": flops / causal_half_flops}

    if not args.no_backward:
        ws = torch.empty(gqa.attn_bwd_workspace_bytes(w.B, w.K, w.G, w.T, w.S, w.H), dtype=torch.uint8, device=dev)
        dq = torch.empty(qd.shape, dtype=torch.float32, device=dev)
        dk = torch.empty(kd.shape, dtype=torch.float32, device=dev)
        dv = torch.empty(vd.shape, dtype=torch.float32, device=dev)
        step()

        def bstep():
            gqa.attn_bwd(qd, kd, vd, o, lse, dod, causal=w.causal, q_seg=segd, kv_seg=segd, dq=dq, dk=dk, dv=dv,
                         workspace=ws)

        try:
            bms = time_launches(bstep, max(5, args.steps // 2), max(2, args.warmup // 2), args.settle_seconds)
            bflops = 2.5 * flops
            result["backward"] = {"ms": bms, "tflops": bflops / (bms * 1e-3) / 1e12,
                                  "frac": bflops / (bms * 1e-3) / 1e12 / MI355X_BF16_DENSE_TFLOPS,
                                  "flops_convention": "2.5x forward (5 matmuls per visible pair)",
                                  "fwd_plus_bwd_tflops": 3.5 * flops / ((ms + bms) * 1e-3) / 1e12}
            kern = {}
            for sub in ("attn_bwd_delta", "attn_bwd_dq", "attn_bwd_dkv"):
                c = measured_counters(w.name, sub)
                if c:
                    kern[sub] = {"mfma_busy": c["mfma_busy"], "clock_ghz": c["clock_ghz"],
                                 "duration_us": c["duration_us"]}
            result["backward"]["kernels"] = kern or None
        except gqa.GqaAttnError as e:
            result["backward"] = {"error": str(e)}

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = n

    if not args.no_cpu_baseline:
        step()
        torch.cuda.synchronize()
        row_flops, okw = None, {"causal": w.causal}
        if seg is not None:
            # a row sees the keys from its segment's start to itself
            starts = np.zeros((w.B, w.T), dtype=np.int64)
            sn = seg.numpy()
            for b in range(w.B):
                idx = np.r_[0, np.flatnonzero(sn[b, 1:] != sn[b, :-1]) + 1]
                starts[b] = idx[np.searchsorted(idx, np.arange(w.T), side="right") - 1]

            def row_flops(rows):
                t = rows % w.T
                b = rows // (w.K * w.G * w.T)
                return float(4.0 * w.H * (t - starts[b, t] + 1).sum())

            okw = {"causal": True, "q_seg": seg, "kv_seg": seg}
        result["cpu_baseline"] = cpu_baseline(inp_cpu, w, o, row_flops=row_flops, oracle_kw=okw, total_flops=flops)
    finish(result)


if __name__ == "__main__":
    main()
