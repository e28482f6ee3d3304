"""Measure the forward's schedule choices per shape class on the local GPU and
write a tuning table in the format of tuning/mi355x.json (with the timings).

For each class, every candidate (load_placement 0/1/2, or a split target) is
timed on the class's representative shapes through attn_fwd_tuned, the
candidates interleaved over several rounds (minimum per candidate), and the
candidate with the smallest geometric-mean time wins. All candidates give
bitwise the same outputs (checked here for the load placements).

Usage (on the GPU): python -m grouped_query_attention_flash_amd.tuning.sweep OUT.json
"""
from __future__ import annotations

import json
import math
import sys
import time

import torch

import grouped_query_attention_flash_amd as gqa
from grouped_query_attention_flash_amd.tuning import gen_table

# (class, table row fields, representative shapes (B, K, G, T, S, H, causal, window_left))
LOAD_PLACEMENT_CLASSES = [
    ("h64_dense", {"H": 64, "segments": 0, "window": 0},
     [(1, 8, 4, 8192, 8192, 64, 1, -1), (2, 8, 4, 4096, 4096, 64, 0, -1)]),
    ("h64_window", {"H": 64, "segments": 0, "window": 1},
     [(1, 8, 4, 8192, 8192, 64, 1, 1023)]),
    ("segments", {"segments": 1},
     [(4, 8, 4, 2048, 2048, 128, 1, "seg"), (4, 8, 4, 2048, 2048, 128, 0, "seg")]),
    ("h128_window", {"H": 128, "segments": 0, "window": 1},
     [(1, 8, 4, 8192, 8192, 128, 1, 1023), (1, 8, 4, 8192, 8192, 128, 1, 4095)]),
    ("h256_dense", {"H": 256, "segments": 0, "window": 0},
     [(1, 2, 8, 32768, 32768, 256, 1, -1), (1, 2, 8, 8192, 8192, 256, 0, -1)]),
    ("h128_dense_causal", {"H": 128, "causal": 1, "segments": 0, "window": 0},
     [(1, 8, 4, 8192, 8192, 128, 1, -1), (2, 8, 4, 4096, 4096, 128, 1, -1)]),
    ("h128_dense_noncausal", {"H": 128, "causal": 0, "segments": 0, "window": 0},
     [(1, 8, 4, 4096, 4096, 128, 0, -1), (1, 1, 4, 256, 256, 128, 0, -1)]),
]
SPLIT_CLASSES = [
    ("decode_h128", {"H": 128, "t_max": 64},
     [(16, 8, 4, 1, 32768, 128, 0, -1), (4, 8, 4, 1, 8192, 128, 0, -1), (16, 8, 4, 4, 8192, 128, 2, -1)]),
    ("decode_h256", {"H": 256, "t_max": 64}, [(8, 2, 8, 1, 32768, 256, 0, -1)]),
    ("decode_h64", {"H": 64, "t_max": 64}, [(16, 8, 4, 1, 16384, 64, 0, -1)]),
    # chunked prefill: a chunk of queries after a long context (few query
    # blocks), split on the ping-pong kernel
    ("prefill_h128", {"H": 128, "t_min": 65},
     [(1, 8, 4, 1024, 8192, 128, 2, -1), (1, 8, 4, 512, 8192, 128, 2, -1), (2, 8, 4, 1024, 8192, 128, 2, -1),
      (1, 8, 4, 256, 8192, 128, 2, -1), (1, 8, 4, 512, 4096, 128, 0, -1)]),
    ("prefill_h64", {"H": 64, "t_min": 65},
     [(1, 8, 4, 1024, 8192, 64, 2, -1), (1, 8, 4, 512, 8192, 64, 2, -1)]),
]
SPLIT_CANDIDATES = [0, 256, 512, 1024, 2048, 4096]


def _timeit(fn, min_s=0.15):
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < 0.1 or n < 2:
        fn()
        torch.cuda.synchronize()
        n += 1
    per = (time.perf_counter() - t0) / n
    steps = max(3, min(100, int(min_s / max(per, 1e-6))))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def _inputs(shape):
    from workloads import make_qkv, make_segment_ids
    B, K, G, T, S, H, causal, win = shape
    q, k, v = (x.cuda() for x in make_qkv(B, K, G, T, S, H, seed=T + S + H))
    kw = {"causal": causal}
    if win == "seg":
        seg = make_segment_ids(B, T, seed=3).cuda()
        kw.update(q_seg=seg, kv_seg=seg.clone())
    elif win >= 0:
        kw["window"] = (win, -1)
    return q, k, v, kw


def sweep_class(shapes, candidates, key, rounds=3):
    """Times per candidate (list over shapes, ms) and the bitwise check."""
    times = {c: [math.inf] * len(shapes) for c in candidates}
    for si, shape in enumerate(shapes):
        q, k, v, kw = _inputs(shape)
        outs = {}
        fns = {}
        for c in candidates:
            # load placements are compared on the single pass (no split)
            lp, st = (c, 0) if key == "load_placement" else (-1, c)
            o = torch.empty_like(q)
            lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
            wsb = gqa.attn_fwd_tuned_workspace_bytes(*shape[:6], st)
            ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=q.device)
            fns[c] = (lambda lp=lp, st=st, o=o, lse=lse, ws=ws: gqa.attn_fwd_tuned(
                q, k, v, load_placement=lp, split_target=st, out=o, lse=lse, workspace=ws, **kw))
            fns[c]()
            torch.cuda.synchronize()
            outs[c] = (o, lse)
        if key == "load_placement":
            o0, l0 = outs[candidates[0]]
            for c in candidates[1:]:
                assert torch.equal(o0, outs[c][0]) and torch.equal(l0, outs[c][1]), (shape, c)
        for _ in range(rounds):
            for c in candidates:
                times[c][si] = min(times[c][si], _timeit(fns[c]))
        print(json.dumps({"shape": list(shape), "ms": {str(c): round(times[c][si], 5) for c in candidates}}),
              flush=True)
    return times


def geomean(xs):
    return math.exp(sum(math.log(x) for x in xs) / len(xs))


def main(out_path):
    table = {"about": json.load(open(gen_table.JSON_PATH))["about"], "load_placement": [], "split_target": []}
    for key, classes, candidates, default in (("load_placement", LOAD_PLACEMENT_CLASSES, [0, 1, 2], 0),
                                              ("split_target", SPLIT_CLASSES, SPLIT_CANDIDATES, 1024)):
        for name, fields, shapes in classes:
            times = sweep_class(shapes, candidates, key)
            best = min(candidates, key=lambda c: geomean(times[c]))
            row = {"class": name, **fields, key: best,
                   "measured": {"shapes": [list(s) for s in shapes],
                                "ms": {str(c): [round(t, 5) for t in times[c]] for c in candidates},
                                "gain_vs_default": round(geomean(times[default]) / geomean(times[best]), 4)}}
            table[key].append(row)
            print(json.dumps({"class": name, key: best, "gain_vs_default": row["measured"]["gain_vs_default"]}),
                  flush=True)
        table[key].append({"class": "default", key: default})
    gen_table.check(table)
    with open(out_path, "w") as f:
        json.dump(table, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else "tuning_sweep.json")
