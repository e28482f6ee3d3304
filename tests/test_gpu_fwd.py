"""GPU forward parity: attn_fwd (HIP, through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import grouped_query_attention_flash_amd as gqa
import oracle
from parity_util import (assert_close_lse, assert_close_o, f32, sample_rows, to_dev)
from workloads import WORKLOADS, HEADLINE, make_qkv, make_segment_ids, make_workload_inputs

pytestmark = pytest.mark.gpu


def run_gpu(q, k, v, causal, q_seg=None, kv_seg=None):
    qd, kd, vd, qs, ks = to_dev(q, k, v, q_seg, kv_seg)
    o, lse = gqa.attn_fwd(qd, kd, vd, causal=causal, q_seg=qs, kv_seg=ks)
    torch.cuda.synchronize()
    return o, lse


# Small cases: several tiles each and ragged tails (B, K, G, T, S, H, causal, seg_len_range)
SMALL = [
    (1, 1, 4, 256, 256, 128, False, None),
    (1, 2, 4, 320, 320, 128, True, None),
    (2, 1, 4, 200, 200, 128, True, None),
    (1, 1, 4, 100, 300, 128, False, None),
    (1, 2, 4, 77, 77, 128, True, (5, 40)),
    (2, 2, 4, 512, 512, 128, True, (16, 200)),
    (1, 1, 3, 130, 130, 128, True, None),
    (1, 2, 8, 256, 256, 128, True, None),
    (1, 3, 1, 96, 160, 128, False, None),
    (1, 1, 12, 64, 64, 128, True, None),
    (1, 1, 4, 1, 1, 128, True, None),
    (1, 1, 4, 1, 700, 128, False, None),
    (1, 2, 4, 192, 192, 64, True, None),
    (1, 1, 4, 150, 150, 64, False, (3, 50)),
    (1, 2, 8, 256, 256, 256, True, None),
    (1, 1, 4, 90, 130, 256, False, None),
    (1, 1, 8, 128, 128, 256, True, (10, 60)),
    # whole key tiles without segment ids (the ping-pong path at H <= 128):
    # one- and two-tile causal blocks, ragged T with G = 1, 2, 8, longer H = 64
    (1, 1, 4, 64, 64, 128, True, None),
    (1, 2, 4, 128, 128, 128, True, None),
    (1, 1, 2, 100, 192, 128, False, None),
    (1, 1, 1, 300, 128, 64, False, None),
    (1, 1, 8, 77, 256, 128, False, None),
    (2, 1, 4, 384, 384, 64, True, None),
    # segment ids on whole key tiles with S <= 8192 (the ping-pong path over
    # each block's list of tiles that share an id): causal packed ids, non-causal
    # independent q / kv ids with ragged T, H = 64, G = 8 (32-query blocks)
    (1, 1, 4, 256, 256, 128, True, (16, 100)),
    (1, 2, 4, 200, 320, 128, False, (20, 90)),
    (1, 1, 4, 128, 128, 64, True, (8, 40)),
    (1, 1, 8, 96, 192, 128, False, (10, 60)),
    # H = 256 with G a multiple of 8 (the ping-pong path at H = 256, 32-key
    # tiles): one- and three-tile causal blocks, G = 16, ragged T
    (2, 1, 8, 32, 32, 256, True, None),
    (1, 1, 8, 96, 96, 256, True, None),
    (1, 1, 16, 64, 64, 256, False, None),
    (1, 1, 8, 50, 96, 256, False, None),
    # segment ids over more than 4096 keys per query block (the kernel reads
    # them from memory instead of its LDS copy) and just under that bound
    (1, 1, 4, 64, 4200, 128, False, (200, 900)),
    (1, 1, 4, 4160, 4160, 128, True, (300, 1200)),
    # H = 256 with G not a multiple of 8 on whole 32-key tiles: the general
    # kernel's DENSE specialisation (4 waves, gw = G heads by 128 / G queries)
    (1, 1, 4, 128, 128, 256, True, None),
    (1, 2, 4, 96, 160, 256, False, None),
    (1, 1, 2, 64, 96, 256, False, None),
    (1, 1, 1, 160, 160, 256, False, None),
    (2, 1, 4, 256, 256, 256, True, None),
    # non-causal segment ids with one or two heads per unit (128- and
    # 256-query blocks on the ping-pong kernel): ids change many times past
    # the block's first 64 queries
    (1, 1, 1, 256, 256, 128, False, (10, 60)),
    (1, 1, 2, 192, 256, 128, False, (10, 60)),
    (1, 2, 1, 300, 512, 128, False, (20, 50)),
    (1, 1, 2, 128, 128, 64, False, (5, 30)),
]


def _id(c):
    B, K, G, T, S, H, causal, seg = c
    return "B%dK%dG%dT%dS%dH%d%s%s" % (B, K, G, T, S, H, "c" if causal else "", "seg" if seg else "")


@pytest.mark.parametrize("case", SMALL, ids=[_id(c) for c in SMALL])
def test_fwd_small_vs_oracle_all_elements(case):
    B, K, G, T, S, H, causal, seg = case
    q, k, v = make_qkv(B, K, G, T, S, H, seed=T * 7 + S + H)
    q_seg = kv_seg = None
    if seg:
        # packed segments with equal q / kv ids (T == S) or independent ids
        q_seg = make_segment_ids(B, T, seed=T, lo=seg[0], hi=seg[1])
        kv_seg = q_seg.clone() if T == S else make_segment_ids(B, S, seed=S, lo=seg[0], hi=seg[1])
    o, lse = run_gpu(q, k, v, causal, q_seg, kv_seg)
    ref_o, ref_lse = oracle.fwd(q, k, v, causal=causal, q_seg=q_seg, kv_seg=kv_seg)
    assert_close_o(f32(o), ref_o)
    assert_close_lse(f32(lse), ref_lse)


@pytest.mark.parametrize("name", list(WORKLOADS) + [HEADLINE.name])
def test_fwd_workload_sampled_rows(name):
    w = WORKLOADS.get(name, HEADLINE)
    inp = make_workload_inputs(w)
    o, lse = run_gpu(inp["q"], inp["k"], inp["v"], w.causal, inp.get("q_seg"), inp.get("kv_seg"))
    rows = sample_rows(w.B, w.K, w.G, w.T, n=384, seed=w.seed)
    ref_o, ref_lse = oracle.fwd(inp["q"], inp["k"], inp["v"], causal=w.causal, q_seg=inp.get("q_seg"),
                                kv_seg=inp.get("kv_seg"), rows=rows)
    rows_t = torch.from_numpy(rows).cuda()
    got_o = o.reshape(-1, w.H).index_select(0, rows_t)
    got_lse = lse.reshape(-1).index_select(0, rows_t)
    assert_close_o(f32(got_o), ref_o, what=name + " O")
    assert_close_lse(f32(got_lse), ref_lse, what=name + " lse")


def test_causal_row_zero_and_segment_starts_bit_exact():
    B, K, G, T, H = 2, 2, 4, 384, 128
    q, k, v = make_qkv(B, K, G, T, T, H, seed=101)
    o, _ = run_gpu(q, k, v, True)
    assert torch.equal(o[:, :, :, 0, :].cpu(), v[:, :, None, 0, :].expand(B, K, G, H))
    seg = make_segment_ids(B, T, seed=5, lo=20, hi=90)
    o, _ = run_gpu(q, k, v, True, seg, seg.clone())
    o = o.cpu()
    for b in range(B):
        starts = [0] + [t for t in range(1, T) if seg[b, t] != seg[b, t - 1]]
        for t in starts:
            assert torch.equal(o[b, :, :, t, :], v[b, :, None, t, :].expand(K, G, H)), (b, t)


def test_zero_q_prefix_means_and_lse():
    B, K, G, T, H = 1, 2, 4, 256, 128
    _, k, v = make_qkv(B, K, G, T, T, H, seed=103)
    q = torch.zeros(B, K, G, T, H, dtype=torch.bfloat16)
    o, lse = run_gpu(q, k, v, True)
    vf = v.double().numpy()
    ref = np.cumsum(vf, axis=2) / np.arange(1, T + 1)[None, None, :, None]
    assert_close_o(f32(o), np.broadcast_to(ref[:, :, None], o.shape))
    np.testing.assert_allclose(f32(lse), np.broadcast_to(np.log(np.arange(1, T + 1)), lse.shape), atol=1e-5)


def test_deterministic_bitwise():
    w = WORKLOADS["segments_causal_b4_k8_g4_t2048_h128"]
    inp = make_workload_inputs(w)
    qd, kd, vd, qs, ks = to_dev(inp["q"], inp["k"], inp["v"], inp["q_seg"], inp["kv_seg"])
    o1, l1 = gqa.attn_fwd(qd, kd, vd, causal=True, q_seg=qs, kv_seg=ks)
    o2, l2 = gqa.attn_fwd(qd, kd, vd, causal=True, q_seg=qs, kv_seg=ks)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_large_logits_stay_finite():
    B, K, G, T, H = 1, 1, 4, 256, 128
    q, k, v = make_qkv(B, K, G, T, T, H, seed=107, q_scale=100.0 / 128 ** 0.5)
    o, lse = run_gpu(q, k, v, True)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    ref_o, ref_lse = oracle.fwd(q, k, v, causal=True)
    assert_close_o(f32(o), ref_o)
    np.testing.assert_allclose(f32(lse), ref_lse, rtol=1e-5, atol=1e-3)


def test_fully_masked_rows_give_zero_and_neg_inf():
    B, K, G, T, S, H = 1, 1, 4, 128, 128, 128
    q, k, v = make_qkv(B, K, G, T, S, H, seed=109)
    q_seg = torch.zeros(B, T, dtype=torch.int32)
    q_seg[:, 64:96] = 7  # id 7 never appears among the keys
    kv_seg = torch.zeros(B, S, dtype=torch.int32)
    o, lse = run_gpu(q, k, v, False, q_seg, kv_seg)
    assert torch.all(o[:, :, :, 64:96] == 0)
    assert torch.all(torch.isneginf(lse[:, :, :, 64:96]))
    ref_o, ref_lse = oracle.fwd(q, k, v, causal=False, q_seg=q_seg, kv_seg=kv_seg)
    assert_close_o(f32(o), ref_o)
    assert_close_lse(f32(lse), ref_lse)


@pytest.mark.parametrize("causal,T", [(False, 192), (True, 256)])
def test_segment_ids_any_int32_values(causal, T):
    # ids need not be sorted, contiguous or small: random draws from a pool with
    # a negative and the largest int32 value, mixed within every tile; batch
    # row 1's queries share no id with any key (O = 0, lse = -inf)
    B, K, G, S, H = 2, 1, 4, 256, 128
    q, k, v = make_qkv(B, K, G, T, S, H, seed=127 + T)
    gen = torch.Generator().manual_seed(127 + T)
    pool = torch.tensor([-5, 3, 2 ** 31 - 1, 40], dtype=torch.int32)
    q_seg = pool[torch.randint(0, 4, (B, T), generator=gen)]
    kv_seg = pool[torch.randint(0, 4, (B, S), generator=gen)]
    q_seg[1] = 99
    o, lse = run_gpu(q, k, v, causal, q_seg, kv_seg)
    assert torch.all(o[1] == 0) and torch.all(torch.isneginf(lse[1]))
    ref_o, ref_lse = oracle.fwd(q, k, v, causal=causal, q_seg=q_seg, kv_seg=kv_seg)
    assert_close_o(f32(o), ref_o)
    assert_close_lse(f32(lse), ref_lse)


def test_lse_optional_and_out_buffer_reused():
    B, K, G, T, H = 1, 1, 4, 128, 128
    q, k, v = to_dev(*make_qkv(B, K, G, T, T, H, seed=113))
    out = torch.full_like(q, 3.0)
    o, lse = gqa.attn_fwd(q, k, v, causal=True, out=out, want_lse=False)
    torch.cuda.synchronize()
    assert lse is None and o.data_ptr() == out.data_ptr()
    ref, _ = oracle.fwd(q.cpu(), k.cpu(), v.cpu(), causal=True)
    assert_close_o(f32(o), ref)
