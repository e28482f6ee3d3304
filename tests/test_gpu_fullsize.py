"""Full-size parity at the workloads' own sizes, in the launch configuration
the bench times, denser than the sampled-row checks:

  forward: every row of at least two whole (b, kv head) units, plus one
  random row in every query block of every head (so every workgroup of the
  grid is checked), against the fp64 oracle, to max-abs 2e-2 / rel-L2 5e-3.
  The 32k-token H = 256 shape has two units in all, 2.2 TFLOP of fp64 oracle
  work: it checks one row in every workgroup plus four whole query blocks
  per head instead.

  backward (causal T = S = 8192 and packed segments): every dQ row of two
  whole units, and dK/dV rows in every kv head."""
import numpy as np
import pytest
import torch

import grouped_query_attention_flash_amd as gqa
import oracle
from parity_util import assert_close_all, assert_close_lse, assert_close_o, f32, to_dev
from workloads import HEADLINE, WORKLOADS, make_qkv, make_workload_inputs

pytestmark = pytest.mark.gpu


def _block_rows(w, bq, rng, whole_units=(), whole_blocks_per_head=0):
    """Flat [B,K,G,T] row indices: one random row per bq-query block of every
    head, every row of the listed units, and every row of some whole blocks."""
    n_blocks = (w.T + bq - 1) // bq
    heads = np.arange(w.B * w.K * w.G)
    starts = np.arange(n_blocks) * bq
    offs = rng.integers(0, bq, size=(len(heads), n_blocks))
    t = np.minimum(starts[None, :] + offs, w.T - 1)
    rows = [(heads[:, None] * w.T + t).ravel()]
    for u in whole_units:
        rows.append(np.arange(u * w.G * w.T, (u + 1) * w.G * w.T))
    if whole_blocks_per_head:
        for blk in np.unique(np.linspace(0, n_blocks - 1, whole_blocks_per_head).astype(int)):
            t0 = blk * bq
            rows.append((heads[:, None] * w.T + np.arange(t0, min(t0 + bq, w.T))[None, :]).ravel())
    return np.unique(np.concatenate(rows))


FWD = [
    # workload, query block size of its launch, whole units, whole blocks per head
    ("causal_b2_k8_g4_t4096_h128", 64, (0, 15), 0),
    ("segments_causal_b4_k8_g4_t2048_h128", 64, (0, 31), 0),
    ("causal_b1_k2_g8_t32768_h256", 32, (), 4),
    # the forward of the T = S = 8192 forward+backward workload is this one
    (HEADLINE.name, 64, (0, 3, 7), 0),
]


@pytest.mark.parametrize("name,bq,units,blocks", FWD, ids=[f[0] for f in FWD])
def test_fwd_full_size_whole_units_and_every_block(name, bq, units, blocks):
    w = WORKLOADS.get(name, HEADLINE)
    inp = make_workload_inputs(w)
    qd, kd, vd, qs, ks = to_dev(inp["q"], inp["k"], inp["v"], inp.get("q_seg"), inp.get("kv_seg"))
    o, lse = gqa.attn_fwd(qd, kd, vd, causal=w.causal, q_seg=qs, kv_seg=ks)
    torch.cuda.synchronize()
    rows = _block_rows(w, bq, np.random.default_rng(w.seed), units, blocks)
    ref_o, ref_lse = oracle.fwd(inp["q"], inp["k"], inp["v"], causal=w.causal, q_seg=inp.get("q_seg"),
                                kv_seg=inp.get("kv_seg"), rows=rows)
    idx = torch.from_numpy(rows).cuda()
    assert_close_o(f32(o.reshape(-1, w.H).index_select(0, idx)), ref_o, what=name + " O")
    assert_close_lse(f32(lse.reshape(-1).index_select(0, idx)), ref_lse, what=name + " lse")
    # and each whole unit on its own
    for u in units:
        sel = (rows >= u * w.G * w.T) & (rows < (u + 1) * w.G * w.T)
        assert_close_o(f32(o.reshape(-1, w.H).index_select(0, idx[torch.from_numpy(sel).cuda()])), ref_o[sel],
                       what="%s unit %d" % (name, u))


def _bwd_check(w, inp, kv_per_head, seed):
    qd, kd, vd, dod, qs, ks = to_dev(inp["q"], inp["k"], inp["v"], inp["do"], inp.get("q_seg"), inp.get("kv_seg"))
    o, lse = gqa.attn_fwd(qd, kd, vd, causal=w.causal, q_seg=qs, kv_seg=ks)
    dq, dk, dv = gqa.attn_bwd(qd, kd, vd, o, lse, dod, causal=w.causal, q_seg=qs, kv_seg=ks)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    n_units = w.B * w.K
    qrows = np.concatenate([np.arange(u * w.G * w.T, (u + 1) * w.G * w.T) for u in (0, n_units - 1)])
    # dK / dV in every kv head: the first and last key of every 1024 and some random keys
    kvrows = np.unique(np.concatenate([
        u * w.S + np.concatenate([np.arange(0, w.S, 1024), np.arange(1023, w.S, 1024),
                                  rng.integers(0, w.S, kv_per_head)]) for u in range(n_units)]))
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["do"], causal=w.causal, q_seg=inp.get("q_seg"),
                     kv_seg=inp.get("kv_seg"), qrows=qrows, kvrows=kvrows)
    dq, dk, dv = f32(dq).reshape(-1, w.H), f32(dk).reshape(-1, w.H), f32(dv).reshape(-1, w.H)
    half = len(qrows) // 2
    assert_close_all([("dQ unit 0", dq[qrows[:half]], ref["dq"][:half]),
                      ("dQ unit %d" % (n_units - 1), dq[qrows[half:]], ref["dq"][half:]),
                      ("dK", dk[kvrows], ref["dk"]), ("dV", dv[kvrows], ref["dv"])])


def test_bwd_full_size_whole_units_and_every_kv_head():
    w = WORKLOADS["causal_fwdbwd_b1_k8_g4_t8192_h128"]
    _bwd_check(w, make_workload_inputs(w), 24, seed=55)


def test_bwd_segments_whole_units_and_every_kv_head():
    w = WORKLOADS["segments_causal_b4_k8_g4_t2048_h128"]
    inp = make_workload_inputs(w)
    inp["do"] = make_qkv(w.B, w.K, w.G, w.T, w.S, w.H, seed=34, with_do=True)[3]
    _bwd_check(w, inp, 32, seed=56)
