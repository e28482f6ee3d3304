"""attn_fwd_noalloc (the forward that keeps its split-KV partials in the
library's static device array) against attn_fwd_mask with a caller workspace,
through the C ABI: bitwise-equal O and lse on two calls in a row, the second
with a smaller input (the array keeps the first call's contents), for shapes
that split the key range and one that does not; oversized shapes are refused
before any launch."""
import ctypes

import pytest
import torch

import grouped_query_attention_flash_amd as gqa
import oracle
from parity_util import assert_close_lse, assert_close_o, f32, to_dev
from workloads import make_qkv

pytestmark = pytest.mark.gpu

P = ctypes.c_void_p
SCRATCH_BYTES = 16 << 20


def _ptr(t):
    return None if t is None else P(t.data_ptr())


def _run_both(B, K, G, T, S, H, causal, wl, wr, prefix, seed):
    q, k, v = make_qkv(B, K, G, T, S, H, seed=seed)
    qd, kd, vd = to_dev(q, k, v)
    lib = gqa.load_library()
    st = P(torch.cuda.current_stream().cuda_stream)
    o_ref = torch.empty_like(qd)
    l_ref = torch.empty(B, K, G, T, dtype=torch.float32, device=qd.device)
    wsb = gqa.attn_fwd_workspace_bytes(B, K, G, T, S, H)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=qd.device)
    rc = lib.attn_fwd_mask(_ptr(qd), _ptr(kd), _ptr(vd), _ptr(o_ref), _ptr(l_ref), None, None, B, K, G, T, S, H,
                           causal, wl, wr, prefix, _ptr(ws), wsb, st)
    assert rc == 0, gqa.attn_strerror(rc)
    o = torch.full_like(qd, 5.0)
    lse = torch.full((B, K, G, T), 5.0, dtype=torch.float32, device=qd.device)
    rc = lib.attn_fwd_noalloc(_ptr(qd), _ptr(kd), _ptr(vd), _ptr(o), _ptr(lse), None, None, B, K, G, T, S, H,
                              causal, wl, wr, prefix, st)
    assert rc == 0, gqa.attn_strerror(rc)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), (B, K, G, T, S, H, causal, wl, wr, prefix)
    return q, k, v, o, lse, wsb


@pytest.mark.parametrize("first,second", [
    # decoding shapes (split-KV), then a smaller one
    ((16, 8, 4, 1, 8192, 128, 0, -1, -1, 0), (2, 2, 4, 1, 2000, 128, 0, -1, -1, 0)),
    ((4, 2, 4, 8, 4096, 128, 2, -1, -1, 0), (1, 1, 4, 3, 1030, 64, 2, 200, -1, 16)),
    ((2, 2, 8, 2, 3000, 256, 0, -1, -1, 0), (1, 1, 8, 1, 900, 256, 1, -1, -1, 0)),
    # a shape that fills the GPU without splitting (no scratch), then a decoding one
    ((1, 16, 4, 2048, 2048, 64, 1, -1, -1, 0), (1, 2, 4, 1, 5000, 128, 0, -1, -1, 0)),
    # two splits, then a smaller decoding shape
    ((1, 2, 4, 512, 512, 128, 1, -1, -1, 0), (1, 1, 4, 1, 3000, 128, 0, -1, -1, 0)),
])
def test_noalloc_equals_workspace_entry_point_twice(first, second):
    wsbs = []
    for i, case in enumerate((first, second)):
        B, K, G, T, S, H, causal, wl, wr, prefix = case
        q, k, v, o, lse, wsb = _run_both(B, K, G, T, S, H, causal, wl, wr, prefix, seed=41 + i + S)
        wsbs.append(wsb)
        ref_o, ref_lse = oracle.fwd(q, k, v, causal=causal, window=(wl, wr), prefix=prefix)
        assert_close_o(f32(o), ref_o)
        assert_close_lse(f32(lse), ref_lse)
    assert wsbs[1] <= SCRATCH_BYTES


def test_noalloc_refuses_oversized_and_bad_masks():
    lib = gqa.load_library()
    q = torch.empty(16, dtype=torch.bfloat16, device="cuda")  # never read: refused before any launch
    st = P(torch.cuda.current_stream().cuda_stream)
    # a decoding batch whose split partials need more than the 16 MiB array
    B, K, G, T, S, H = 1, 8, 4, 64, 32768, 128
    assert gqa.attn_fwd_workspace_bytes(B, K, G, T, S, H) > SCRATCH_BYTES
    args = (_ptr(q), _ptr(q), _ptr(q), _ptr(q), None, None, None, B, K, G, T, S, H)
    assert lib.attn_fwd_noalloc(*args, 0, -1, -1, 0, st) == gqa.GQA_ATTN_ERR_WORKSPACE
    assert lib.attn_fwd_noalloc(*args, 3, -1, -1, 0, st) == gqa.GQA_ATTN_ERR_MASK
    assert lib.attn_fwd_noalloc(*args, 1, -1, -1, -4, st) == gqa.GQA_ATTN_ERR_MASK
    torch.cuda.synchronize()


def test_noalloc_binding():
    B, K, G, T, S, H = 4, 2, 4, 2, 6000, 128
    q, k, v = make_qkv(B, K, G, T, S, H, seed=7)
    qd, kd, vd = to_dev(q, k, v)
    o = torch.empty_like(qd)
    lse = torch.empty(B, K, G, T, dtype=torch.float32, device=qd.device)
    gqa.attn_fwd_noalloc(qd, kd, vd, o, lse, causal=2)
    o2, l2 = gqa.attn_fwd(qd, kd, vd, causal=2, split_kv=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)
