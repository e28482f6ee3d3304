"""GPU parity of the split-KV forward (attn_fwd_ws) against the fp64 oracle.

Shapes with few query rows per kv head (decoding, T << S) split the key range
across workgroups; every case here checks that the split path is taken
(attn_fwd_split_count > 1) before comparing all elements of O and lse with
the oracle, to the same bar as the plain forward."""
import numpy as np
import pytest
import torch

import grouped_query_attention_flash_amd as gqa
import oracle
from parity_util import assert_close_lse, assert_close_o, f32, to_dev
from workloads import make_qkv, make_segment_ids

pytestmark = pytest.mark.gpu


def run_split(q, k, v, causal, q_seg=None, kv_seg=None, workspace=None):
    qd, kd, vd, qs, ks = to_dev(q, k, v, q_seg, kv_seg)
    o, lse = gqa.attn_fwd(qd, kd, vd, causal=causal, q_seg=qs, kv_seg=ks, split_kv=True, workspace=workspace)
    torch.cuda.synchronize()
    return o, lse


# (B, K, G, T, S, H, causal, seg_len_range): decode and short-query shapes,
# ragged S, every head size, causal (top-left: most splits see no key), segments.
# Up to 16 query rows per (b, kv head) without a mask take the decoding kernel
# (the rows of all heads in one 16-column tile, 16-key tiles per wave): R = 1,
# 4, 8, 12 and 16, H = 64, 128 and 256, a last split of 9 keys (its other
# waves see none).
CASES = [
    (1, 2, 4, 1, 4096, 128, False, None),
    (2, 2, 4, 3, 3000, 128, False, None),
    (1, 1, 8, 1, 1030, 64, False, None),
    (1, 2, 4, 16, 4096, 128, True, None),
    (1, 1, 4, 5, 2500, 256, False, None),
    (1, 2, 4, 4, 4096, 128, False, (100, 900)),
    (1, 1, 1, 1, 2048, 128, False, None),
    (1, 1, 4, 40, 8000, 128, False, None),
    (2, 2, 8, 2, 5000, 128, False, None),
    (1, 2, 4, 4, 3000, 64, False, None),
    (3, 1, 2, 1, 1289, 128, False, None),
    (1, 2, 8, 1, 3000, 256, False, None),
    (2, 1, 4, 4, 2000, 256, False, None),
]


def _id(c):
    B, K, G, T, S, H, causal, seg = c
    return "B%dK%dG%dT%dS%dH%d%s%s" % (B, K, G, T, S, H, "c" if causal else "", "seg" if seg else "")


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_split_kv_vs_oracle_all_elements(case):
    B, K, G, T, S, H, causal, seg = case
    assert gqa.attn_fwd_split_count(B, K, G, T, S, H) > 1, "shape does not take the split path"
    q, k, v = make_qkv(B, K, G, T, S, H, seed=T * 11 + S + H)
    q_seg = kv_seg = None
    if seg:
        # ids shared by the query rows and a run of keys; the queries' ids are
        # the keys' ids at the query positions, so every query sees some keys
        kv_seg = make_segment_ids(B, S, seed=S, lo=seg[0], hi=seg[1])
        q_seg = kv_seg[:, S - T:].clone().contiguous()
    o, lse = run_split(q, k, v, causal, q_seg, kv_seg)
    ref_o, ref_lse = oracle.fwd(q, k, v, causal=causal, q_seg=q_seg, kv_seg=kv_seg)
    assert_close_o(f32(o), ref_o)
    assert_close_lse(f32(lse), ref_lse)


def test_split_kv_matches_single_pass():
    """The split and single-pass forwards agree to fp32 summation-order
    differences (the merge is exact in real arithmetic)."""
    B, K, G, T, S, H = 1, 2, 4, 2, 6144, 128
    q, k, v = make_qkv(B, K, G, T, S, H, seed=5)
    o_s, lse_s = run_split(q, k, v, False)
    qd, kd, vd = to_dev(q, k, v)
    o_1, lse_1 = gqa.attn_fwd(qd, kd, vd, causal=False)
    torch.cuda.synchronize()
    assert float((o_s.float() - o_1.float()).abs().max()) <= 1.6e-2  # bf16 rounding of O either side
    np.testing.assert_allclose(f32(lse_s), f32(lse_1), rtol=0, atol=1e-4)


def test_split_kv_rows_without_visible_keys():
    """A row whose id matches no key: every split reports lse = -inf, and the
    merge gives O = 0 and lse = -inf."""
    B, K, G, T, S, H = 1, 1, 4, 4, 4096, 128
    q, k, v = make_qkv(B, K, G, T, S, H, seed=17)
    kv_seg = torch.zeros(B, S, dtype=torch.int32)
    q_seg = torch.zeros(B, T, dtype=torch.int32)
    q_seg[:, 1] = 9
    o, lse = run_split(q, k, v, False, q_seg, kv_seg)
    assert torch.all(o[:, :, :, 1] == 0)
    assert torch.all(torch.isneginf(lse[:, :, :, 1]))
    ref_o, ref_lse = oracle.fwd(q, k, v, causal=False, q_seg=q_seg, kv_seg=kv_seg)
    assert_close_o(f32(o), ref_o)
    assert_close_lse(f32(lse), ref_lse)


def test_split_kv_workspace_reused_across_calls():
    """Two calls in a row on one workspace, the second with a smaller shape,
    each against the oracle."""
    ws = torch.empty(gqa.attn_fwd_workspace_bytes(1, 2, 4, 1, 8192, 128), dtype=torch.uint8, device="cuda")
    for (B, K, G, T, S, H) in [(1, 2, 4, 1, 8192, 128), (1, 1, 4, 1, 3000, 128)]:
        assert gqa.attn_fwd_workspace_bytes(B, K, G, T, S, H) <= ws.numel()
        q, k, v = make_qkv(B, K, G, T, S, H, seed=S)
        o, lse = run_split(q, k, v, False, workspace=ws)
        ref_o, ref_lse = oracle.fwd(q, k, v, causal=False)
        assert_close_o(f32(o), ref_o)
        assert_close_lse(f32(lse), ref_lse)
