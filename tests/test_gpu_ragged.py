"""GPU parity of the ping-pong forward on key lengths that are not a whole
number of its key tiles: the partial last tile loads with range-checked
per-lane offsets and its keys at or past S are masked. Every element of O and
lse against the fp64 oracle, through the single pass (split_target 0)."""
import pytest
import torch

import grouped_query_attention_flash_amd as gqa
import oracle
from parity_util import assert_close_lse, assert_close_o, f32, to_dev
from workloads import make_qkv

pytestmark = pytest.mark.gpu

# (B, K, G, T, S, H, causal, window_left)
CASES = [
    (1, 2, 4, 1000, 1000, 128, 1, -1),  # top-left causal, T = S
    (2, 2, 4, 65, 65, 128, 1, -1),  # a one-key last tile
    (1, 2, 4, 333, 333, 64, 1, -1),
    (1, 1, 8, 100, 100, 256, 1, -1),  # 32-key tiles at H = 256
    (1, 1, 8, 77, 200, 256, 0, -1),
    (1, 2, 4, 100, 1124, 128, 2, -1),  # end-aligned: a 100-query chunk after 1024 keys
    (1, 1, 4, 300, 700, 128, 0, -1),  # non-causal, partial tile of 60 keys
    (1, 1, 4, 1, 1000, 128, 0, -1),  # one query row
    (1, 1, 4, 1000, 1000, 128, 1, 100),  # causal left window
    (4, 8, 4, 1000, 1000, 128, 1, -1),  # more blocks than compute units
]


def _id(c):
    return "B%dK%dG%dT%dS%dH%dc%d_w%d" % c


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_partial_key_tile_vs_oracle_all_elements(case):
    B, K, G, T, S, H, causal, wl = case
    q, k, v = make_qkv(B, K, G, T, S, H, seed=T * 3 + S + H)
    qd, kd, vd = to_dev(q, k, v)
    kw = {"causal": causal, "split_target": 0}
    if wl >= 0:
        kw["window"] = (wl, -1)
    o, lse = gqa.attn_fwd_tuned(qd, kd, vd, **kw)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.fwd(q, k, v, causal=causal, window=(wl, -1) if wl >= 0 else None)
    assert_close_o(f32(o), ref_o)
    assert_close_lse(f32(lse), ref_lse)


def test_partial_key_tile_placements_agree():
    """Explicit M-phase load placements fall back to the V-phase one on a
    partial last tile: bitwise the same result."""
    q, k, v = to_dev(*make_qkv(1, 2, 4, 300, 300, 64, seed=17))
    ref = gqa.attn_fwd_tuned(q, k, v, causal=1, load_placement=0, split_target=0)
    for lp in (1, 2):
        got = gqa.attn_fwd_tuned(q, k, v, causal=1, load_placement=lp, split_target=0)
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), lp
