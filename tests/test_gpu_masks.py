"""GPU parity of the end-aligned causal mask (causal=2: s <= t + S - T) and of
prefix keys (s < p visible to every query), through attn_fwd / attn_bwd and
attn_fwd_mask / attn_bwd_mask, against the fp64 oracle's visibility rule.

Every element of O, lse, dQ, dK and dV is compared at sizes that span several
key and query tiles with ragged tails; chunked-prefill shapes (a block of new
queries after a long context) are compared on sampled rows at full size. The
shapes reach each kernel family: the ping-pong forward at H = 64, 128 and 256
(a diagonal offset of whole tiles), the general kernels (ragged or offset
tiles, prefixes), and the split-KV forward (few query rows)."""
import ctypes

import numpy as np
import pytest
import torch

import grouped_query_attention_flash_amd as gqa
import oracle
from parity_util import assert_close_all, assert_close_lse, assert_close_o, f32, sample_rows, to_dev
from workloads import make_qkv, make_segment_ids

pytestmark = pytest.mark.gpu

# (B, K, G, T, S, H, causal, window, prefix, segments)
FWD_CASES = [
    # end-aligned causal: new queries after S - T context keys
    (1, 1, 4, 256, 2048, 128, 2, None, 0, False),   # offset 1792 = 28 tiles of 64
    (1, 2, 4, 128, 1024, 64, 2, None, 0, False),
    (1, 1, 8, 96, 512, 256, 2, None, 0, False),     # offset 416 = 13 tiles of 32
    (1, 1, 4, 100, 300, 128, 2, None, 0, False),    # ragged
    (1, 1, 4, 300, 100, 128, 2, None, 0, False),    # T > S: the first 200 rows see nothing
    (2, 1, 3, 77, 200, 128, 2, None, 0, True),
    (1, 1, 4, 192, 1000, 128, 2, (64, -1), 0, False),
    (1, 1, 4, 256, 288, 128, 2, None, 0, False),    # offset 32: not a whole 64-key tile
    # prefix keys
    (1, 2, 4, 256, 256, 128, 1, None, 100, False),
    (1, 1, 4, 320, 320, 64, 1, None, 64, False),
    (1, 1, 4, 200, 200, 256, 1, None, 37, False),
    (1, 1, 8, 128, 128, 256, 1, None, 70, False),
    (1, 1, 4, 512, 512, 128, 1, (63, -1), 16, False),  # a few global keys and a causal band
    (2, 1, 4, 160, 160, 128, 1, None, 50, True),
    (1, 1, 4, 130, 400, 128, 2, None, 20, False),
    (1, 1, 4, 200, 200, 128, 0, (10, 10), 5, False),
    (1, 1, 2, 64, 5000, 128, 1, None, 300, False),    # few query rows: the split-KV path
]


def _id(c):
    B, K, G, T, S, H, causal, win, pfx, seg = c
    w = "" if win is None else "_w%d_%d" % win
    return "B%dK%dG%dT%dS%dH%d_c%d%s_p%d%s" % (B, K, G, T, S, H, causal, w, pfx, "seg" if seg else "")


def _segments(B, T, S, seg):
    if not seg:
        return None, None
    q_seg = make_segment_ids(B, T, seed=T, lo=10, hi=60)
    return q_seg, q_seg.clone() if T == S else make_segment_ids(B, S, seed=S, lo=10, hi=60)


def _mask_kw(causal, win, pfx):
    kw = {"causal": causal}
    if win is not None:
        kw["window"] = win
    if pfx:
        kw["prefix"] = pfx
    return kw


@pytest.mark.parametrize("case", FWD_CASES, ids=[_id(c) for c in FWD_CASES])
def test_mask_fwd_vs_oracle_all_elements(case):
    B, K, G, T, S, H, causal, win, pfx, seg = case
    q, k, v = make_qkv(B, K, G, T, S, H, seed=T * 11 + S + H + pfx)
    q_seg, kv_seg = _segments(B, T, S, seg)
    qd, kd, vd, qs, ks = to_dev(q, k, v, q_seg, kv_seg)
    kw = _mask_kw(causal, win, pfx)
    o, lse = gqa.attn_fwd(qd, kd, vd, q_seg=qs, kv_seg=ks, **kw)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.fwd(q, k, v, q_seg=q_seg, kv_seg=kv_seg, **kw)
    assert_close_o(f32(o), ref_o)
    assert_close_lse(f32(lse), ref_lse)


BWD_CASES = FWD_CASES


@pytest.mark.parametrize("case", BWD_CASES, ids=[_id(c) for c in BWD_CASES])
def test_mask_bwd_vs_oracle_all_elements(case):
    B, K, G, T, S, H, causal, win, pfx, seg = case
    q, k, v, do = make_qkv(B, K, G, T, S, H, seed=T * 13 + S + H + pfx, with_do=True)
    q_seg, kv_seg = _segments(B, T, S, seg)
    qd, kd, vd, dod, qs, ks = to_dev(q, k, v, do, q_seg, kv_seg)
    kw = _mask_kw(causal, win, pfx)
    o, lse = gqa.attn_fwd(qd, kd, vd, q_seg=qs, kv_seg=ks, **kw)
    dq, dk, dv = gqa.attn_bwd(qd, kd, vd, o, lse, dod, q_seg=qs, kv_seg=ks, **kw)
    torch.cuda.synchronize()
    ref = oracle.bwd(q, k, v, do, q_seg=q_seg, kv_seg=kv_seg, **kw)
    assert_close_all([("dQ", f32(dq), ref["dq"]), ("dK", f32(dk), ref["dk"]), ("dV", f32(dv), ref["dv"])])


@pytest.mark.parametrize("T", [128, 512, 1024])
def test_end_aligned_chunked_prefill_full_size_sampled(T):
    """B=1, K=8, G=4, S=8192, H=128: T new queries at the end of the context,
    end-aligned causal, forward and backward on sampled rows (every query
    block's first and last row of two kv heads, and random rows)."""
    B, K, G, S, H = 1, 8, 4, 8192, 128
    q, k, v, do = make_qkv(B, K, G, T, S, H, seed=T + 17, with_do=True)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    o, lse = gqa.attn_fwd(qd, kd, vd, causal=2)
    dq, dk, dv = gqa.attn_bwd(qd, kd, vd, o, lse, dod, causal=2)
    torch.cuda.synchronize()
    rows = sample_rows(B, K, G, T, n=256, seed=T)
    ref_o, ref_lse = oracle.fwd(q, k, v, causal=2, rows=rows)
    assert_close_o(f32(o.reshape(-1, H)[torch.from_numpy(rows).cuda()]), ref_o)
    assert_close_lse(f32(lse.reshape(-1)[torch.from_numpy(rows).cuda()]), ref_lse)
    units = [0, K - 1]
    rng = np.random.default_rng(T)
    qrows = np.unique(np.concatenate([u * G * T + sample_rows(1, 1, G, T, 32, seed=u) for u in units]))
    kvrows = np.unique(np.concatenate([u * S + np.concatenate([[0, S - T - 1, S - T, S - 1], rng.integers(0, S, 48)])
                                       for u in units]))
    ref = oracle.bwd(q, k, v, do, causal=2, qrows=qrows, kvrows=kvrows)
    assert_close_all([("dQ", f32(dq).reshape(-1, H)[qrows], ref["dq"]),
                      ("dK", f32(dk).reshape(-1, H)[kvrows], ref["dk"]),
                      ("dV", f32(dv).reshape(-1, H)[kvrows], ref["dv"])])


@pytest.mark.parametrize("T,S", [(1, 32768), (4, 4096), (16, 2000)])
def test_end_aligned_decode_split_kv(T, S):
    """Few queries at the end of a long context through the split-KV forward
    (attn_fwd_ws); with T = 1 every key is visible (the non-causal result)."""
    B, K, G, H = 2, 2, 4, 128
    q, k, v = make_qkv(B, K, G, T, S, H, seed=S + T)
    qd, kd, vd = to_dev(q, k, v)
    assert gqa.attn_fwd_split_count(B, K, G, T, S, H) > 1
    o, lse = gqa.attn_fwd(qd, kd, vd, causal=2, split_kv=True)
    o1, lse1 = gqa.attn_fwd(qd, kd, vd, causal=2)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.fwd(q, k, v, causal=2)
    assert_close_o(f32(o), ref_o)
    assert_close_lse(f32(lse), ref_lse)
    assert_close_o(f32(o1), ref_o)
    if T == 1:
        ref_n, _ = oracle.fwd(q, k, v, causal=False)
        assert np.array_equal(ref_n, ref_o)


def test_huge_window_sides_equal_unbounded():
    """Window sides far beyond the sequence (up to INT_MAX) bound nothing: the
    result is bitwise that of the unwindowed call, forward and backward."""
    B, K, G, T, H = 1, 2, 4, 256, 128
    q, k, v, do = to_dev(*make_qkv(B, K, G, T, T, H, seed=131, with_do=True))
    big = 2 ** 31 - 1
    for causal, win in ((False, (big, big)), (True, (big, -1)), (False, (-1, big)), (True, (big, big))):
        o0, l0 = gqa.attn_fwd(q, k, v, causal=causal)
        o1, l1 = gqa.attn_fwd(q, k, v, causal=causal, window=win)
        g0 = gqa.attn_bwd(q, k, v, o0, l0, do, causal=causal)
        g1 = gqa.attn_bwd(q, k, v, o1, l1, do, causal=causal, window=win)
        torch.cuda.synchronize()
        assert torch.equal(o0, o1) and torch.equal(l0, l1), (causal, win)
        for a, b in zip(g0, g1):
            assert torch.equal(a, b), (causal, win)
    # and a huge side next to a real one still matches the oracle
    o, lse = gqa.attn_fwd(q, k, v, causal=False, window=(big, 40))
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.fwd(q.cpu(), k.cpu(), v.cpu(), causal=False, window=(-1, 40))
    assert_close_o(f32(o), ref_o)
    assert_close_lse(f32(lse), ref_lse)


def test_local_entry_points_equal_mask_entry_points():
    """attn_fwd_local / attn_bwd_local are attn_fwd_mask / attn_bwd_mask with
    prefix 0: bitwise the same outputs."""
    B, K, G, T, S, H = 1, 1, 4, 192, 256, 128
    q, k, v, do = to_dev(*make_qkv(B, K, G, T, S, H, seed=137, with_do=True))
    lib = gqa.load_library()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = ctypes.c_void_p
    o_a, o_b = torch.empty_like(q), torch.empty_like(q)
    l_a = torch.empty(B, K, G, T, device=q.device)
    l_b = torch.empty_like(l_a)
    args = lambda o, l: (P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(o.data_ptr()), P(l.data_ptr()),
                         None, None, B, K, G, T, S, H, 1)
    assert lib.attn_fwd_local(*args(o_a, l_a), 50, -1, None, 0, st) == 0
    assert lib.attn_fwd_mask(*args(o_b, l_b), 50, -1, 0, None, 0, st) == 0
    ws = torch.empty(gqa.attn_bwd_workspace_bytes(B, K, G, T, S, H), dtype=torch.uint8, device=q.device)
    grads = []
    for fn in ("attn_bwd_local", "attn_bwd_mask"):
        dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
        dv = torch.empty_like(dk)
        extra = (50, -1) if fn == "attn_bwd_local" else (50, -1, 0)
        rc = getattr(lib, fn)(P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), None, P(l_a.data_ptr()),
                              P(do.data_ptr()), P(dq.data_ptr()), P(dk.data_ptr()), P(dv.data_ptr()), None, None,
                              B, K, G, T, S, H, 1, *extra, P(ws.data_ptr()), ws.numel(), st)
        assert rc == 0, fn
        grads.append((dq, dk, dv))
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(l_a, l_b)
    for a, b in zip(*grads):
        assert torch.equal(a, b)
