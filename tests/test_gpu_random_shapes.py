"""GPU parity over a seeded random sweep of small shapes and masks, through
every dispatch path of the forward (ping-pong dense, ragged and persistent;
split-KV on the ping-pong, decoding and general kernels; the general kernel)
and of the backward (ping-pong D and dQ, wave-pair and general dK/dV).
Every element of O and lse, or of dQ, dK and dV, against the fp64 oracle.

The cases are drawn once from a fixed seed: half of them on whole 64-key
tiles, where the fast paths apply, half on arbitrary T and S; head dims 64,
128 and 256; G from 1 to 8; the three causal modes; and no mask, a window,
a prefix or segment ids."""
import numpy as np
import pytest
import torch

import grouped_query_attention_flash_amd as gqa
import oracle
from parity_util import assert_close_all, assert_close_lse, assert_close_o, f32, to_dev
from workloads import make_qkv, make_segment_ids

pytestmark = pytest.mark.gpu


def _draw(n, seed, fwd):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        H = int(rng.choice([64, 128, 256]))
        G = int(rng.choice([1, 2, 3, 4, 8]))
        B, K = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        if rng.random() < 0.5:
            T = 64 * int(rng.integers(1, 5))
            S = T if rng.random() < 0.6 else 64 * int(rng.integers(1, 5))
        else:
            T, S = int(rng.integers(1, 260)), int(rng.integers(1, 260))
        causal = int(rng.choice([0, 1, 2]))
        mask = str(rng.choice(["none", "window", "prefix", "segments"], p=[0.5, 0.2, 0.1, 0.2]))
        wl = wr = -1
        prefix = 0
        if mask == "window":
            wl = int(rng.integers(0, 200))
            wr = -1 if causal else int(rng.choice([-1, int(rng.integers(0, 100))]))
        elif mask == "prefix":
            prefix = int(rng.integers(1, S + 1))
        split = fwd and bool(rng.random() < 0.5)
        cases.append((B, K, G, T, S, H, causal, mask, wl, wr, prefix, split))
    return cases


FWD = _draw(96, 20261203, True)
BWD = _draw(48, 31122026, False)


def _id(c):
    B, K, G, T, S, H, causal, mask, wl, wr, prefix, split = c
    return "B%dK%dG%dT%dS%dH%d_c%d_%s%s%s" % (
        B, K, G, T, S, H, causal, mask, "_w%d,%d" % (wl, wr) if mask == "window" else "",
        "_p%d" % prefix if mask == "prefix" else "") + ("_split" if split else "")


def _inputs(c, with_do):
    B, K, G, T, S, H, causal, mask, wl, wr, prefix, split = c
    t = make_qkv(B, K, G, T, S, H, seed=T * 7 + S * 3 + H + G, with_do=with_do)
    q_seg = kv_seg = None
    if mask == "segments":
        q_seg = make_segment_ids(B, T, seed=T + S, lo=8, hi=96)
        kv_seg = q_seg.clone() if T == S else make_segment_ids(B, S, seed=T + S + 1, lo=8, hi=96)
    return t, q_seg, kv_seg


def _mask_kw(c):
    B, K, G, T, S, H, causal, mask, wl, wr, prefix, split = c
    kw = {"causal": causal}
    if mask == "window":
        kw["window"] = (wl, wr)
    if mask == "prefix":
        kw["prefix"] = prefix
    return kw


def _oracle_kw(c, q_seg, kv_seg):
    kw = _mask_kw(c)
    if q_seg is not None:
        kw["q_seg"], kw["kv_seg"] = q_seg, kv_seg
    return kw


@pytest.mark.parametrize("case", FWD, ids=[_id(c) for c in FWD])
def test_fwd_random_shape_vs_oracle(case):
    (q, k, v), q_seg, kv_seg = _inputs(case, False)
    qd, kd, vd, qs, ks = to_dev(q, k, v, q_seg, kv_seg)
    o, lse = gqa.attn_fwd(qd, kd, vd, q_seg=qs, kv_seg=ks, split_kv=case[-1], **_mask_kw(case))
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.fwd(q, k, v, **_oracle_kw(case, q_seg, kv_seg))
    assert_close_o(f32(o), ref_o)
    assert_close_lse(f32(lse), ref_lse)


@pytest.mark.parametrize("case", BWD, ids=[_id(c) for c in BWD])
def test_bwd_random_shape_vs_oracle(case):
    (q, k, v, do), q_seg, kv_seg = _inputs(case, True)
    qd, kd, vd, dod, qs, ks = to_dev(q, k, v, do, q_seg, kv_seg)
    kw = _mask_kw(case)
    o, lse = gqa.attn_fwd(qd, kd, vd, q_seg=qs, kv_seg=ks, **kw)
    dq, dk, dv = gqa.attn_bwd(qd, kd, vd, o, lse, dod, q_seg=qs, kv_seg=ks, **kw)
    torch.cuda.synchronize()
    ref = oracle.bwd(q, k, v, do, **_oracle_kw(case, q_seg, kv_seg))
    assert_close_all([("dQ", f32(dq), ref["dq"]), ("dK", f32(dk), ref["dk"]), ("dV", f32(dv), ref["dv"])])
