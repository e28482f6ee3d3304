"""GPU backward parity: attn_bwd (HIP, through the C ABI) against the fp64 oracle.

The gradients are fp32; the pair max-abs 2e-2 / rel-L2 5e-3 applies to each
of dQ, dK and dV. The GPU recomputes P from its own forward's lse and rounds
P and dS to bf16 as MFMA operands; the oracle does neither."""
import numpy as np
import pytest
import torch

import grouped_query_attention_flash_amd as gqa
import oracle
from parity_util import assert_close_all, sample_rows, to_dev
from workloads import WORKLOADS, make_qkv, make_segment_ids, make_workload_inputs

pytestmark = pytest.mark.gpu


def run_gpu(q, k, v, do, causal, q_seg=None, kv_seg=None):
    qd, kd, vd, dod, qs, ks = to_dev(q, k, v, do, q_seg, kv_seg)
    o, lse = gqa.attn_fwd(qd, kd, vd, causal=causal, q_seg=qs, kv_seg=ks)
    dq, dk, dv = gqa.attn_bwd(qd, kd, vd, o, lse, dod, causal=causal, q_seg=qs, kv_seg=ks)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


SMALL = [
    (1, 1, 4, 256, 256, 128, False, None),
    (1, 2, 4, 320, 320, 128, True, None),
    (2, 1, 4, 200, 200, 128, True, None),
    (1, 1, 4, 100, 300, 128, False, None),
    (1, 1, 4, 100, 300, 128, True, None),  # causal with S > T: keys past T - 1 see no query
    (1, 2, 4, 130, 200, 64, True, None),
    (1, 2, 4, 160, 160, 128, True, (5, 40)),
    (2, 1, 4, 384, 384, 128, True, (16, 200)),
    (1, 1, 3, 130, 130, 128, True, None),
    (1, 1, 8, 128, 128, 128, True, None),
    (1, 2, 1, 96, 160, 128, False, None),
    (1, 1, 4, 1, 1, 128, True, None),
    (1, 2, 4, 192, 192, 64, True, None),
    (1, 1, 4, 128, 128, 256, True, None),
    (1, 1, 4, 90, 130, 256, False, (3, 50)),
    # dense shapes of the ping-pong D pass: non-causal with T != S, and
    # one and two heads per unit (256- and 128-query blocks of the dense dQ path)
    (1, 1, 1, 256, 256, 128, True, None),
    (1, 2, 2, 256, 384, 128, False, None),
    # eight heads per unit (32-query blocks)
    (1, 1, 4, 128, 320, 128, False, None),
    (1, 1, 8, 96, 128, 128, False, None),
    (1, 1, 4, 64, 192, 64, False, None),
]


def _id(c):
    B, K, G, T, S, H, causal, seg = c
    return "B%dK%dG%dT%dS%dH%d%s%s" % (B, K, G, T, S, H, "c" if causal else "", "seg" if seg else "")


@pytest.mark.parametrize("case", SMALL, ids=[_id(c) for c in SMALL])
def test_bwd_small_vs_oracle_all_elements(case):
    B, K, G, T, S, H, causal, seg = case
    q, k, v, do = make_qkv(B, K, G, T, S, H, seed=T * 3 + S + H, with_do=True)
    q_seg = kv_seg = None
    if seg:
        q_seg = make_segment_ids(B, T, seed=T, lo=seg[0], hi=seg[1])
        kv_seg = q_seg.clone() if T == S else make_segment_ids(B, S, seed=S, lo=seg[0], hi=seg[1])
    dq, dk, dv = run_gpu(q, k, v, do, causal, q_seg, kv_seg)
    ref = oracle.bwd(q, k, v, do, causal=causal, q_seg=q_seg, kv_seg=kv_seg)
    assert_close_all([("dQ", dq, ref["dq"]), ("dK", dk, ref["dk"]), ("dV", dv, ref["dv"])])


def test_bwd_dq_with_and_without_the_ds_lo_part():
    """Causal T = S = 2048 at H = 128 (the ping-pong dQ kernel): waves of the
    early rows see |dS| above the bound for adding dS's bf16 lo part into dQ,
    waves of the later rows stay under it and drop it. Every element of dQ,
    dK and dV against the oracle."""
    q, k, v, do = make_qkv(1, 1, 4, 2048, 2048, 128, seed=2048, with_do=True)
    dq, dk, dv = run_gpu(q, k, v, do, True)
    ref = oracle.bwd(q, k, v, do, causal=True)
    assert_close_all([("dQ", dq, ref["dq"]), ("dK", dk, ref["dk"]), ("dV", dv, ref["dv"])])
    # the first and last 256 rows of every head separately: both paths pass
    dq4, ref4 = dq.reshape(4, 2048, 128), ref["dq"].reshape(4, 2048, 128)
    assert_close_all([("dQ rows 0-255", dq4[:, :256], ref4[:, :256]),
                      ("dQ rows 1792-2047", dq4[:, -256:], ref4[:, -256:])])


def test_bwd_fwdbwd_workload_sampled_rows():
    """B=1, K=8, G=4, T=S=8192, H=128, causal: sampled dQ rows and dK/dV rows of two kv heads."""
    w = WORKLOADS["causal_fwdbwd_b1_k8_g4_t8192_h128"]
    inp = make_workload_inputs(w)
    dq, dk, dv = run_gpu(inp["q"], inp["k"], inp["v"], inp["do"], w.causal)
    rng = np.random.default_rng(5)
    units = [0, w.K - 1]
    qrows = np.unique(np.concatenate([u * w.G * w.T + sample_rows(1, 1, w.G, w.T, 96, seed=u) for u in units]))
    kvrows = np.unique(np.concatenate([u * w.S + np.concatenate([[0, 1, w.S - 1], rng.integers(0, w.S, 96)])
                                       for u in units]))
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["do"], causal=True, qrows=qrows, kvrows=kvrows)
    assert_close_all([("dQ", dq.reshape(-1, w.H)[qrows], ref["dq"]),
                      ("dK", dk.reshape(-1, w.H)[kvrows], ref["dk"]),
                      ("dV", dv.reshape(-1, w.H)[kvrows], ref["dv"])])


def test_bwd_segments_workload_sampled_rows():
    w = WORKLOADS["segments_causal_b4_k8_g4_t2048_h128"]
    inp = make_workload_inputs(w)
    inp["do"] = make_qkv(w.B, w.K, w.G, w.T, w.S, w.H, seed=33, with_do=True)[3]
    dq, dk, dv = run_gpu(inp["q"], inp["k"], inp["v"], inp["do"], True, inp["q_seg"], inp["kv_seg"])
    units = [0, 13, w.B * w.K - 1]
    qrows = np.unique(np.concatenate([u * w.G * w.T + sample_rows(1, 1, w.G, w.T, 64, seed=u) for u in units]))
    rng = np.random.default_rng(3)
    kvrows = np.unique(np.concatenate([u * w.S + rng.integers(0, w.S, 64) for u in units]))
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["do"], causal=True, q_seg=inp["q_seg"],
                     kv_seg=inp["kv_seg"], qrows=qrows, kvrows=kvrows)
    assert_close_all([("dQ", dq.reshape(-1, w.H)[qrows], ref["dq"]),
                      ("dK", dk.reshape(-1, w.H)[kvrows], ref["dk"]),
                      ("dV", dv.reshape(-1, w.H)[kvrows], ref["dv"])])


def test_bwd_invariants_and_determinism():
    B, K, G, T, H = 1, 2, 4, 512, 128
    q, k, v, do = make_qkv(B, K, G, T, T, H, seed=77, with_do=True)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    o, lse = gqa.attn_fwd(qd, kd, vd, causal=True)
    r1 = gqa.attn_bwd(qd, kd, vd, o, lse, dod, causal=True)
    r2 = gqa.attn_bwd(qd, kd, vd, o, lse, dod, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    dq, dk, dv = (x.double().cpu().numpy() for x in r1)
    # sum_s dS[t, s] = 0 -> sum_s dK = 0, up to the rounding of P, dS
    assert np.abs(dk.sum(axis=2)).max() <= 2e-3 * np.abs(dk).sum(axis=2).max()
    # rows of P sum to 1 -> sum_s dV = sum_{g,t} dO, up to bf16 P
    ref = do.double().numpy().sum(axis=(2, 3))
    assert np.abs(dv.sum(axis=2) - ref).max() <= 5e-3 * np.abs(ref).max() + 1e-2


def test_bwd_fully_masked_rows_get_zero_gradient():
    B, K, G, T, H = 1, 1, 4, 128, 128
    q, k, v, do = make_qkv(B, K, G, T, T, H, seed=79, with_do=True)
    q_seg = torch.zeros(B, T, dtype=torch.int32)
    q_seg[:, 32:64] = 9  # never present among the keys
    kv_seg = torch.zeros(B, T, dtype=torch.int32)
    dq, dk, dv = run_gpu(q, k, v, do, False, q_seg, kv_seg)
    assert np.all(dq[:, :, :, 32:64] == 0)
    assert np.all(np.isfinite(dq)) and np.all(np.isfinite(dk)) and np.all(np.isfinite(dv))
    ref = oracle.bwd(q, k, v, do, causal=False, q_seg=q_seg, kv_seg=kv_seg)
    assert_close_all([("dQ", dq, ref["dq"]), ("dK", dk, ref["dk"]), ("dV", dv, ref["dv"])])


def test_bwd_workspace_too_small_is_rejected():
    B, K, G, T, H = 1, 1, 4, 64, 128
    q, k, v, do = to_dev(*make_qkv(B, K, G, T, T, H, seed=81, with_do=True))
    o, lse = gqa.attn_fwd(q, k, v, causal=True)
    ws = torch.empty(16, dtype=torch.uint8, device=q.device)
    with pytest.raises(gqa.GqaAttnError) as ei:
        gqa.attn_bwd(q, k, v, o, lse, do, causal=True, workspace=ws)
    assert ei.value.code == gqa.GQA_ATTN_ERR_WORKSPACE
