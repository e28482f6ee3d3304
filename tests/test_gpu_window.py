"""GPU parity of the local-window forward and backward (attn_fwd_local,
attn_bwd_local) against the fp64 oracle's band rule t - wl <= s <= t + wr.

Every element of O, lse, dQ, dK and dV is compared, to the same bar as the
unwindowed paths, on shapes that span several key and query tiles with
ragged tails, both window sides, causal and non-causal, every head size,
segment ids, and a decoding shape that takes the split-KV path."""
import numpy as np
import pytest
import torch

import grouped_query_attention_flash_amd as gqa
import oracle
from parity_util import assert_close_all, assert_close_lse, assert_close_o, f32, to_dev
from workloads import make_qkv, make_segment_ids

pytestmark = pytest.mark.gpu

# (B, K, G, T, S, H, causal, wl, wr, segments)
CASES = [
    (1, 2, 4, 256, 256, 128, True, 63, -1, False),
    (1, 1, 4, 300, 300, 128, True, 100, -1, False),
    (1, 2, 4, 200, 260, 128, False, 40, 30, False),
    (1, 1, 8, 128, 128, 64, True, 0, -1, False),
    (1, 1, 4, 160, 160, 256, True, 50, -1, False),
    (1, 2, 4, 192, 192, 128, True, 31, -1, True),
    (2, 1, 4, 96, 333, 128, False, -1, 70, False),
    (1, 1, 4, 100, 300, 128, True, 37, -1, False),
    # causal left windows on whole 64-key tiles, T == S: the ping-pong kernel
    # from each block's first visible tile (cut first tile, single-tile blocks)
    (1, 2, 4, 512, 512, 128, True, 127, -1, False),
    (1, 1, 4, 448, 448, 128, True, 100, -1, False),
    (1, 1, 4, 256, 256, 128, True, 20, -1, False),
    (1, 2, 4, 384, 384, 64, True, 191, 5, False),
]


def _id(c):
    B, K, G, T, S, H, causal, wl, wr, seg = c
    return "B%dK%dG%dT%dS%dH%d%s_w%d_%d%s" % (B, K, G, T, S, H, "c" if causal else "", wl, wr, "seg" if seg else "")


def _segments(B, T, S, seg):
    if not seg:
        return None, None
    q_seg = make_segment_ids(B, T, seed=T, lo=20, hi=90)
    return q_seg, q_seg.clone() if T == S else make_segment_ids(B, S, seed=S, lo=20, hi=90)


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_window_fwd_vs_oracle_all_elements(case):
    B, K, G, T, S, H, causal, wl, wr, seg = case
    q, k, v = make_qkv(B, K, G, T, S, H, seed=T * 5 + S + H + wl)
    q_seg, kv_seg = _segments(B, T, S, seg)
    qd, kd, vd, qs, ks = to_dev(q, k, v, q_seg, kv_seg)
    o, lse = gqa.attn_fwd(qd, kd, vd, causal=causal, q_seg=qs, kv_seg=ks, window=(wl, wr))
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.fwd(q, k, v, causal=causal, q_seg=q_seg, kv_seg=kv_seg, window=(wl, wr))
    assert_close_o(f32(o), ref_o)
    assert_close_lse(f32(lse), ref_lse)


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_window_bwd_vs_oracle_all_elements(case):
    B, K, G, T, S, H, causal, wl, wr, seg = case
    q, k, v, do = make_qkv(B, K, G, T, S, H, seed=T * 3 + S + H + wl, with_do=True)
    q_seg, kv_seg = _segments(B, T, S, seg)
    qd, kd, vd, dod, qs, ks = to_dev(q, k, v, do, q_seg, kv_seg)
    o, lse = gqa.attn_fwd(qd, kd, vd, causal=causal, q_seg=qs, kv_seg=ks, window=(wl, wr))
    dq, dk, dv = gqa.attn_bwd(qd, kd, vd, o, lse, dod, causal=causal, q_seg=qs, kv_seg=ks, window=(wl, wr))
    torch.cuda.synchronize()
    ref = oracle.bwd(q, k, v, do, causal=causal, q_seg=q_seg, kv_seg=kv_seg, window=(wl, wr))
    assert_close_all([("dQ", f32(dq), ref["dq"]), ("dK", f32(dk), ref["dk"]), ("dV", f32(dv), ref["dv"])])


def test_window_split_kv_decoding():
    """A short-query shape with a right-bounded window: the split-KV path
    (several splits see no key at all) against the oracle."""
    B, K, G, T, S, H, wl, wr = 1, 2, 4, 8, 4096, 128, -1, 1000
    assert gqa.attn_fwd_split_count(B, K, G, T, S, H) > 1
    q, k, v = make_qkv(B, K, G, T, S, H, seed=97)
    qd, kd, vd = to_dev(q, k, v)
    o, lse = gqa.attn_fwd(qd, kd, vd, causal=False, window=(wl, wr))
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.fwd(q, k, v, causal=False, window=(wl, wr))
    assert_close_o(f32(o), ref_o)
    assert_close_lse(f32(lse), ref_lse)


def test_unbounded_window_equals_plain_calls():
    """window=(-1, -1) is the plain forward / backward, bit for bit on the
    general kernels."""
    B, K, G, T, S, H = 1, 1, 4, 100, 300, 128
    q, k, v, do = make_qkv(B, K, G, T, S, H, seed=101, with_do=True)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    o0, l0 = gqa.attn_fwd(qd, kd, vd, causal=False)
    o1, l1 = gqa.attn_fwd(qd, kd, vd, causal=False, window=(-1, -1))
    g0 = gqa.attn_bwd(qd, kd, vd, o0, l0, dod, causal=False)
    g1 = gqa.attn_bwd(qd, kd, vd, o1, l1, dod, causal=False, window=(-1, -1))
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)
