"""GPU parity of split-KV on the ping-pong forward (dense shapes without a
window, H <= 128): each split covers part of every query block's key tiles,
only the split holding a block's diagonal tile masks it, splits that miss a
block's keys contribute nothing, and the merge combines them. Every element
of O and lse against the fp64 oracle, with splits forced by an explicit
split target."""
import pytest
import torch

import grouped_query_attention_flash_amd as gqa
import oracle
from parity_util import assert_close_lse, assert_close_o, f32, to_dev
from workloads import make_qkv

pytestmark = pytest.mark.gpu

# (B, K, G, T, S, H, causal, split_target)
CASES = [
    (1, 2, 4, 256, 2048, 128, 2, 1024),  # chunked prefill: 256 queries after 1792 keys
    (1, 2, 4, 512, 512, 128, 1, 1024),  # top-left causal: early blocks leave later splits empty
    (1, 2, 4, 128, 3000, 128, 0, 1024),  # non-causal, partial last key tile
    (2, 2, 4, 130, 1154, 128, 2, 4096),  # ragged T and S, end-aligned
    (1, 1, 4, 100, 1124, 64, 2, 1024),
    (1, 2, 8, 96, 2048, 128, 0, 1024),  # G = 8: 32-query blocks of 8 heads
]


def _id(c):
    return "B%dK%dG%dT%dS%dH%dc%d_st%d" % c


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_pp_split_vs_oracle_all_elements(case):
    B, K, G, T, S, H, causal, target = case
    assert gqa.attn_fwd_tuned_workspace_bytes(B, K, G, T, S, H, target) > 0, "the call does not split"
    q, k, v = make_qkv(B, K, G, T, S, H, seed=T * 5 + S + H)
    qd, kd, vd = to_dev(q, k, v)
    o, lse = gqa.attn_fwd_tuned(qd, kd, vd, causal=causal, split_target=target)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.fwd(q, k, v, causal=causal)
    assert_close_o(f32(o), ref_o)
    assert_close_lse(f32(lse), ref_lse)
    # and the single pass on the same tensors, to the same bar
    o1, lse1 = gqa.attn_fwd_tuned(qd, kd, vd, causal=causal, split_target=0)
    torch.cuda.synchronize()
    assert_close_o(f32(o), f32(o1), what="split vs single pass O")
    assert_close_lse(f32(lse), f32(lse1), what="split vs single pass lse")
