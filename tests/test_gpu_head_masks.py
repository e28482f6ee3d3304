"""GPU parity of per-head masks (attn_fwd_head_masks, attn_bwd_head_masks):
every query head (k, g) takes its own window sides and prefix from a device
table, as the splash baseline's MultiHeadMask gives each head its own mask
(danielwatson6.github.io/fa, "Our first kernel"). The oracle needs nothing
new: each head is one oracle call on that head's slice with its own mask, and
the heads' dK / dV contributions add up. Every element against the oracle."""
import numpy as np
import pytest
import torch

import grouped_query_attention_flash_amd as gqa
import oracle
from parity_util import assert_close_all, assert_close_lse, assert_close_o, f32, to_dev
from workloads import make_qkv, make_segment_ids

pytestmark = pytest.mark.gpu

GLOBAL, LOCAL64, LOCAL128_P16, DIAG = (-1, -1, 0), (63, -1, 0), (127, -1, 16), (0, -1, 0)
TWO_SIDED, PREFIX_ONLY, BAND = (40, 25, 0), (-1, 10, 50), (7, 7, 3)

# (B, K, G, T, S, H, causal, segments, per-head (wl, wr, prefix) rows cycled over the K*G heads)
CASES = [
    (1, 2, 4, 256, 256, 128, 1, False, [GLOBAL, LOCAL64, LOCAL128_P16, DIAG]),
    (1, 1, 4, 200, 300, 64, 0, False, [TWO_SIDED, PREFIX_ONLY, BAND, GLOBAL]),
    (2, 1, 8, 96, 320, 128, 2, False, [LOCAL64, GLOBAL, (15, -1, 200), DIAG]),
    (1, 1, 8, 128, 128, 256, 1, False, [GLOBAL, LOCAL64, (31, -1, 0), LOCAL128_P16]),
    (1, 1, 4, 192, 192, 128, 1, True, [GLOBAL, LOCAL64, LOCAL128_P16, DIAG]),
    # values the kernels normalise: any negative side unbounded, a prefix past
    # S, sides past the sequence
    (1, 2, 2, 130, 130, 128, 1, False, [(-7, -3, 0), (10, -1, 1000), (5000, 5000, 0), (3, 4, -9)]),
    (1, 1, 3, 64, 64, 64, 0, False, [(0, 0, 0), GLOBAL, (5, 0, 8)]),
    # shapes of the ping-pong D and dQ kernels and the wave-pair dK/dV kernel
    # (whole tiles, causal T = S): per-wave masks over the union of a block's heads
    (1, 2, 4, 512, 512, 128, 1, False, [GLOBAL, (255, -1, 0), (63, -1, 32), DIAG]),
    (1, 1, 4, 384, 384, 64, 0, False, [TWO_SIDED, PREFIX_ONLY, BAND, (100, 30, 20)]),
    # (a prefix of only 3 keys under a 5-key window would gather about 1500 of
    # the eight heads' bf16-rounded weights on each of those keys: that
    # rounding alone, which the kernels share with the pages' fused kernel,
    # moves dV there by 2.1e-2, past the absolute bar; with 40 prefix keys it
    # is 1.3e-2, as a CPU simulation of bf16 weights in fp64 shows)
    (2, 1, 8, 256, 256, 128, 1, False, [GLOBAL, (31, -1, 0), (127, -1, 64), DIAG, (0, -1, 200), LOCAL64,
                                        GLOBAL, (5, -1, 40)]),
    (1, 1, 2, 256, 320, 128, 0, False, [(50, 50, 0), (-1, -1, 100)]),
]


def _id(c):
    return "B%dK%dG%dT%dS%dH%d_c%d%s" % (c[:7] + ("_seg" if c[7] else "",))


def _table(K, G, rows):
    t = np.array([rows[i % len(rows)] for i in range(K * G)], dtype=np.int32).reshape(K, G, 3)
    return t


def _oracle_kw(row, causal):
    wl, wr, pfx = (int(x) for x in row)
    return {"causal": causal, "window": (wl if wl >= 0 else -1, wr if wr >= 0 else -1), "prefix": max(pfx, 0)}


def _inputs(c, with_do):
    B, K, G, T, S, H, causal, segs, rows = c
    t = make_qkv(B, K, G, T, S, H, seed=T * 11 + S + G, with_do=with_do)
    q_seg = kv_seg = None
    if segs:
        q_seg = make_segment_ids(B, T, seed=T, lo=16, hi=80)
        kv_seg = q_seg.clone()
    return t, q_seg, kv_seg


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_fwd_head_masks_vs_oracle(case):
    B, K, G, T, S, H, causal, segs, rows = case
    (q, k, v), q_seg, kv_seg = _inputs(case, False)
    table = _table(K, G, rows)
    qd, kd, vd, qs, ks = to_dev(q, k, v, q_seg, kv_seg)
    o, lse = gqa.attn_fwd(qd, kd, vd, causal=causal, q_seg=qs, kv_seg=ks,
                          head_mask=torch.from_numpy(table).cuda())
    torch.cuda.synchronize()
    ref_o = np.zeros((B, K, G, T, H))
    ref_lse = np.zeros((B, K, G, T))
    for kh in range(K):
        for g in range(G):
            kw = _oracle_kw(table[kh, g], causal)
            if segs:
                kw["q_seg"], kw["kv_seg"] = q_seg, kv_seg
            o1, l1 = oracle.fwd(q[:, kh:kh + 1, g:g + 1], k[:, kh:kh + 1], v[:, kh:kh + 1], **kw)
            ref_o[:, kh, g] = o1[:, 0, 0]
            ref_lse[:, kh, g] = l1[:, 0, 0]
    assert_close_o(f32(o), ref_o)
    assert_close_lse(f32(lse), ref_lse)


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_bwd_head_masks_vs_oracle(case):
    B, K, G, T, S, H, causal, segs, rows = case
    (q, k, v, do), q_seg, kv_seg = _inputs(case, True)
    table = torch.from_numpy(_table(K, G, rows))
    qd, kd, vd, dod, qs, ks = to_dev(q, k, v, do, q_seg, kv_seg)
    hm = table.cuda()
    o, lse = gqa.attn_fwd(qd, kd, vd, causal=causal, q_seg=qs, kv_seg=ks, head_mask=hm)
    dq, dk, dv = gqa.attn_bwd(qd, kd, vd, o, lse, dod, causal=causal, q_seg=qs, kv_seg=ks, head_mask=hm)
    torch.cuda.synchronize()
    ref_dq = np.zeros((B, K, G, T, H))
    ref_dk = np.zeros((B, K, S, H))
    ref_dv = np.zeros((B, K, S, H))
    for kh in range(K):
        for g in range(G):
            kw = _oracle_kw(table[kh, g].numpy(), causal)
            if segs:
                kw["q_seg"], kw["kv_seg"] = q_seg, kv_seg
            r = oracle.bwd(q[:, kh:kh + 1, g:g + 1], k[:, kh:kh + 1], v[:, kh:kh + 1], do[:, kh:kh + 1, g:g + 1],
                           **kw)
            ref_dq[:, kh, g] = r["dq"][:, 0, 0]
            ref_dk[:, kh] += r["dk"][:, 0]
            ref_dv[:, kh] += r["dv"][:, 0]
    assert_close_all([("dQ", f32(dq), ref_dq), ("dK", f32(dk), ref_dk), ("dV", f32(dv), ref_dv)])


def test_uniform_table_matches_the_single_mask_call():
    """A table with the same mask on every head gives the single-mask call's
    result (through the general kernels instead of the fast paths)."""
    B, K, G, T, S, H = 1, 2, 4, 256, 256, 128
    q, k, v, do = to_dev(*make_qkv(B, K, G, T, S, H, seed=5, with_do=True))
    hm = torch.tensor([[[100, -1, 8]] * G] * K, dtype=torch.int32).cuda()
    o1, l1 = gqa.attn_fwd(q, k, v, causal=True, head_mask=hm)
    o2, l2 = gqa.attn_fwd(q, k, v, causal=True, window=(100, -1), prefix=8)
    g1 = gqa.attn_bwd(q, k, v, o1, l1, do, causal=True, head_mask=hm)
    g2 = gqa.attn_bwd(q, k, v, o2, l2, do, causal=True, window=(100, -1), prefix=8)
    torch.cuda.synchronize()
    assert_close_o(f32(o1), f32(o2), what="O per-head vs single mask")
    assert_close_lse(f32(l1), f32(l2), what="lse per-head vs single mask")
    assert_close_all([("dQ", f32(g1[0]), f32(g2[0])), ("dK", f32(g1[1]), f32(g2[1])), ("dV", f32(g1[2]), f32(g2[2]))])


def test_head_mask_binding_refusals():
    """Bad table tensors are refused before anything is launched."""
    q, k, v = to_dev(*make_qkv(1, 2, 4, 64, 64, 128, seed=1))
    good = torch.zeros(2, 4, 3, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        gqa.attn_fwd(q, k, v, head_mask=good.to(torch.int64))
    with pytest.raises(ValueError):
        gqa.attn_fwd(q, k, v, head_mask=good[:, :3])
    with pytest.raises(ValueError):
        gqa.attn_fwd(q, k, v, head_mask=good.cpu())
    with pytest.raises(ValueError):
        gqa.attn_fwd(q, k, v, head_mask=good, window=(4, -1))
