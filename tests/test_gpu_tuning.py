"""attn_fwd_tuned: every explicit schedule choice computes the forward the
library's own choice does. Load placements are bitwise equal to attn_fwd;
split targets (which change only how the key range is cut and merged) match
the fp64 oracle; out-of-range choices are refused before any launch."""
import pytest
import torch

import grouped_query_attention_flash_amd as gqa
import oracle
from parity_util import assert_close_lse, assert_close_o, f32, to_dev
from workloads import make_qkv, make_segment_ids

pytestmark = pytest.mark.gpu

# (B, K, G, T, S, H, causal, window_left, segments): each reaches the ping-pong kernel
PP_SHAPES = [
    (1, 2, 4, 512, 512, 128, 1, -1, False),
    (1, 1, 4, 256, 384, 128, 0, -1, False),
    (1, 2, 4, 384, 384, 64, 1, -1, False),
    (1, 1, 8, 256, 256, 256, 1, -1, False),
    (2, 1, 4, 512, 512, 128, 1, -1, True),
    (1, 1, 4, 512, 512, 128, 1, 100, False),
]


@pytest.mark.parametrize("shape", PP_SHAPES)
def test_load_placements_are_bitwise_equal(shape):
    B, K, G, T, S, H, causal, wl, seg = shape
    q, k, v = to_dev(*make_qkv(B, K, G, T, S, H, seed=T + H + wl))
    kw = {"causal": causal}
    if seg:
        s_ids = make_segment_ids(B, T, seed=9, lo=30, hi=150).cuda()
        kw.update(q_seg=s_ids, kv_seg=s_ids.clone())
    if wl >= 0:
        kw["window"] = (wl, -1)
    # split_target 0: the single pass (no split-KV), whatever the mask
    o_ref, l_ref = gqa.attn_fwd_tuned(q, k, v, load_placement=0, split_target=0, **kw)
    if wl < 0:
        o_p, l_p = gqa.attn_fwd(q, k, v, **kw)  # attn_fwd never splits
        torch.cuda.synchronize()
        assert torch.equal(o_p, o_ref) and torch.equal(l_p, l_ref), shape
    for lp in (1, 2):
        o, lse = gqa.attn_fwd_tuned(q, k, v, load_placement=lp, split_target=0, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), (shape, lp)


@pytest.mark.parametrize("split_target", [0, 256, 1024, 4096])
def test_split_targets_match_the_oracle(split_target):
    B, K, G, T, S, H = 4, 2, 4, 2, 6000, 128
    q, k, v = make_qkv(B, K, G, T, S, H, seed=split_target + 1)
    qd, kd, vd = to_dev(q, k, v)
    o, lse = gqa.attn_fwd_tuned(qd, kd, vd, split_target=split_target, causal=2)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.fwd(q, k, v, causal=2)
    assert_close_o(f32(o), ref_o)
    assert_close_lse(f32(lse), ref_lse)


def test_tuned_refuses_bad_choices():
    q, k, v = to_dev(*make_qkv(1, 1, 4, 64, 64, 128, seed=3))
    out = torch.full_like(q, 2.0)
    for bad in (dict(load_placement=3), dict(load_placement=-2), dict(split_target=-5),
                dict(split_target=(1 << 20) + 1)):
        with pytest.raises(gqa.GqaAttnError) as e:
            gqa.attn_fwd_tuned(q, k, v, out=out, **bad)
        assert e.value.code == gqa.GQA_ATTN_ERR_TUNING
    torch.cuda.synchronize()
    assert bool((out == 2.0).all())
