"""GPU parity of the ping-pong forward's persistent grid.

A dense call at H <= 128 with more query blocks than compute units runs one
workgroup per compute unit, each walking several blocks; with loads in the
softmax phase each block also loads the next one's Q and first tiles and the
blocks rotate the LDS slots. A call over one batch row of the same tensors
has few enough blocks to launch one workgroup per block, and every block
computes the same arithmetic either way, so the two must agree bit for bit.
Sampled rows are also checked against the fp64 oracle."""
import pytest
import torch

import grouped_query_attention_flash_amd as gqa
import oracle
from parity_util import assert_close_lse, assert_close_o, f32, sample_rows, to_dev
from workloads import make_qkv

pytestmark = pytest.mark.gpu

# (B, K, G, T, S, H, causal, window_left): B * K * T / 64 blocks, well past
# 256, except the last (264 blocks: a few workgroups take a second block)
CASES = [
    (8, 8, 4, 1024, 1024, 128, 1, -1),
    (8, 8, 4, 1000, 1024, 128, 0, -1),  # ragged last query block
    (16, 8, 4, 512, 1024, 128, 2, -1),  # end-aligned causal, S > T
    (8, 8, 4, 1024, 1024, 128, 1, 100),  # causal left window
    (8, 8, 4, 1024, 1024, 64, 1, -1),
    (3, 8, 4, 704, 704, 128, 1, -1),
    (8, 8, 4, 1000, 1000, 128, 0, -1),  # partial last key tile
    (8, 8, 4, 1000, 1000, 128, 1, -1),
]


def _id(c):
    return "B%dK%dG%dT%dS%dH%dc%d_w%d" % c


def _call(q, k, v, causal, wl):
    # split_target 0: the single pass, also for a window (whose calls would
    # otherwise split the key range of a small grid)
    kw = {"causal": causal, "split_target": 0}
    if wl >= 0:
        kw["window"] = (wl, -1)
    return gqa.attn_fwd_tuned(q, k, v, **kw)


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_persistent_grid_equals_per_block_launch(case):
    B, K, G, T, S, H, causal, wl = case
    q, k, v = make_qkv(B, K, G, T, S, H, seed=B * 1000 + T + H + wl)
    qd, kd, vd = to_dev(q, k, v)
    o, lse = _call(qd, kd, vd, causal, wl)
    torch.cuda.synchronize()
    for b in range(B):
        ob, lb = _call(qd[b:b + 1].contiguous(), kd[b:b + 1].contiguous(), vd[b:b + 1].contiguous(), causal, wl)
        torch.cuda.synchronize()
        assert torch.equal(ob[0], o[b]) and torch.equal(lb[0], lse[b]), (case, b)
    rows = sample_rows(B, K, G, T, n=1024, seed=T + B)
    ref_o, ref_lse = oracle.fwd(q, k, v, causal=causal, rows=rows, window=(wl, -1) if wl >= 0 else None)
    rows_t = torch.from_numpy(rows).cuda()
    assert_close_o(f32(o.reshape(-1, H).index_select(0, rows_t)), ref_o)
    assert_close_lse(f32(lse.reshape(-1).index_select(0, rows_t)), ref_lse)
