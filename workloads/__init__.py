"""Seeded synthetic inputs for grouped-query attention.

This module is shared by the tests, the bench and the oracle's callers. It
holds no attention arithmetic: it only draws random tensors, pre-scales the
queries (the op itself applies no scale) and builds segment-id arrays.

Notation (page "Notation", danielwatson6.github.io/fa): B batch, T queries,
S keys/values, K kv heads, G query heads per kv head, H head dim. Queries are
laid out [B, K, G, T, H]; keys and values [B, K, S, H]. Queries arrive already
multiplied by H^-1/2 (same page, "What is wrong with naive attention?").

Recipe:
  * a CPU ``torch.Generator`` seeded with ``seed`` draws fp32 N(0, 1) tensors
    in the order q, k, v, dO;
  * q is multiplied by H^-1/2 in fp32;
  * every tensor is rounded once to bf16 (round to nearest even);
  * segment ids use a second generator seeded with ``seed + 1000``: per batch
    row, segment lengths are drawn uniformly from [lo, hi] (inclusive) until
    they cover T; the last segment is cut to fit; ids count 0, 1, 2, ... and
    the kv ids equal the q ids (packed sequences, T == S).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    K: int
    G: int
    T: int
    S: int
    H: int
    causal: bool
    segments: bool
    backward: bool
    seed: int


# The five workloads: shapes, masks and seeds.
WORKLOADS = {
    "noncausal_b1_k1_g4_t256_h128": Workload(
        "noncausal_b1_k1_g4_t256_h128", 1, 1, 4, 256, 256, 128, False, False, False, 1),
    "causal_b2_k8_g4_t4096_h128": Workload(
        "causal_b2_k8_g4_t4096_h128", 2, 8, 4, 4096, 4096, 128, True, False, False, 2),
    "segments_causal_b4_k8_g4_t2048_h128": Workload(
        "segments_causal_b4_k8_g4_t2048_h128", 4, 8, 4, 2048, 2048, 128, True, True, False, 3),
    "causal_b1_k2_g8_t32768_h256": Workload(
        "causal_b1_k2_g8_t32768_h256", 1, 2, 8, 32768, 32768, 256, True, False, False, 4),
    "causal_fwdbwd_b1_k8_g4_t8192_h128": Workload(
        "causal_fwdbwd_b1_k8_g4_t8192_h128", 1, 8, 4, 8192, 8192, 128, True, False, True, 5),
}

# The headline forward: 32 query heads over 8 kv heads, T = S = 8192, H = 128,
# causal (same tensors as the forward+backward workload, seed 5).
HEADLINE = dataclasses.replace(
    WORKLOADS["causal_fwdbwd_b1_k8_g4_t8192_h128"],
    name="causal_b1_k8_g4_t8192_h128", backward=False)


# Decoding: one query row per head (T = 1) against a 32768-token context, the
# regime where the intensity is about G FLOP per byte and the forward is bound
# by reading K and V. Not one of the five workloads; bench.py times it with
# --workload decode.
DECODE = Workload("decode_b16_k8_g4_t1_s32768_h128", 16, 8, 4, 1, 32768, 128, False, False, False, 6)


# Sliding window: the headline shape with a causal band of 1024 keys (each
# query sees itself and the 1023 keys before it). bench.py --workload window.
WINDOW = Workload("window1024_causal_b1_k8_g4_t8192_h128", 1, 8, 4, 8192, 8192, 128, True, False, True, 7)
WINDOW_LEFT = 1023


# Chunked prefill: a chunk of 1024 new queries at the end of an 8192-token
# context (7168 cached keys), end-aligned causal (query t sees keys
# s <= t + S - T). One workgroup per 256 query rows gives only 128 blocks, so
# the call splits the key range. bench.py --workload prefill.
PREFILL = Workload("prefill_endcausal_b1_k8_g4_t1024_s8192_h128", 1, 8, 4, 1024, 8192, 128, True, False, False, 8)
PREFILL_CAUSAL = 2  # the end-aligned form of the causal argument


def workload_by_bench_name(name: str) -> Workload:
    """The workload bench.py's --workload option names."""
    return {"headline": HEADLINE, "decode": DECODE, "window": WINDOW, "prefill": PREFILL,
            "long": WORKLOADS["causal_b1_k2_g8_t32768_h256"],
            "segments": WORKLOADS["segments_causal_b4_k8_g4_t2048_h128"]}[name]


def window_pairs(T: int, S: int, wl: int, causal: bool = True) -> int:
    """Visible (t, s) pairs per head of a causal band t - wl <= s <= t."""
    assert causal
    return sum(min(t, S - 1) - max(0, t - wl) + 1 for t in range(T) if t - wl <= S - 1)


def end_aligned_pairs(T: int, S: int) -> int:
    """Visible (t, s) pairs per head when query t sees keys s <= t + S - T."""
    return sum(max(0, min(S, t + S - T + 1)) for t in range(T))


def make_qkv(B: int, K: int, G: int, T: int, S: int, H: int, seed: int,
             with_do: bool = False, q_scale: Optional[float] = None):
    """Draw q, k, v (and dO) as bf16 CPU tensors, contiguous, H innermost."""
    gen = torch.Generator().manual_seed(seed)
    q = torch.randn(B, K, G, T, H, generator=gen, dtype=torch.float32)
    k = torch.randn(B, K, S, H, generator=gen, dtype=torch.float32)
    v = torch.randn(B, K, S, H, generator=gen, dtype=torch.float32)
    do = torch.randn(B, K, G, T, H, generator=gen, dtype=torch.float32) if with_do else None
    scale = float(H) ** -0.5 if q_scale is None else q_scale
    q = q * scale
    out = [q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)]
    if with_do:
        out.append(do.to(torch.bfloat16))
    return tuple(out)


def make_segment_ids(B: int, T: int, seed: int, lo: int = 64, hi: int = 1024):
    """Nondecreasing int32 segment ids [B, T] with lengths ~ UniformInt[lo, hi]."""
    gen = torch.Generator().manual_seed(seed + 1000)
    ids = torch.empty(B, T, dtype=torch.int32)
    for b in range(B):
        pos, sid = 0, 0
        while pos < T:
            n = int(torch.randint(lo, hi + 1, (1,), generator=gen).item())
            n = min(n, T - pos)
            ids[b, pos:pos + n] = sid
            pos += n
            sid += 1
    return ids


def make_workload_inputs(w: Workload):
    """All inputs of a workload: dict with q, k, v, [do], [q_seg, kv_seg]."""
    t = make_qkv(w.B, w.K, w.G, w.T, w.S, w.H, w.seed, with_do=w.backward)
    d = {"q": t[0], "k": t[1], "v": t[2]}
    if w.backward:
        d["do"] = t[3]
    if w.segments:
        assert w.T == w.S
        seg = make_segment_ids(w.B, w.T, w.seed)
        d["q_seg"] = seg
        d["kv_seg"] = seg.clone()
    return d


def attention_flops(B: int, K: int, G: int, T: int, S: int, H: int, causal: bool) -> float:
    """Forward FLOPs: 4*B*K*G*T*S*H (two matmuls), halved when causal (T == S)."""
    f = 4.0 * B * K * G * T * S * H
    return f / 2.0 if causal else f


def visible_pairs_flops(H: int, K: int, G: int, seg_ids, causal: bool = True) -> float:
    """Forward FLOPs counting only visible (t, s) pairs of packed causal segments."""
    total = 0
    for b in range(seg_ids.shape[0]):
        _, counts = torch.unique_consecutive(seg_ids[b], return_counts=True)
        for n in counts.tolist():
            total += n * (n + 1) // 2 if causal else n * n
    return 4.0 * H * K * G * total
