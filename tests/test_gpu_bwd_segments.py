"""GPU parity of the backward with segment ids (SegmentIds of the fjformer
page; the FA page's splash kernel takes them too): the wave-pair dK/dV
kernel walks only the query tiles whose ids meet its keys' ids, the
ping-pong D and dQ kernels only the key tiles whose ids meet their queries',
and all three mask pairs of different ids element by element. Every element
of dQ, dK and dV against the fp64 oracle, with ids packed in order, ids in
no order at all, blocks that meet no id, and each mask form the ids combine
with (the shapes that the ping-pong kernels do not take run the general
ones)."""
import numpy as np
import pytest
import torch

import grouped_query_attention_flash_amd as gqa
import oracle
from parity_util import assert_close_all, f32, to_dev
from workloads import make_qkv, make_segment_ids

pytestmark = pytest.mark.gpu


def _scattered_ids(B, T, seed, values):
    """int32 ids drawn independently per position from `values`: the tiles'
    id ranges overlap everywhere and most pairs need the element mask."""
    rng = np.random.default_rng(seed)
    return torch.from_numpy(rng.choice(np.array(values, dtype=np.int32), size=(B, T)))


# (B, K, G, T, S, H, causal, ids, extra mask keywords)
CASES = [
    (1, 2, 4, 640, 640, 128, 1, ("packed", 16, 200), {}),
    (2, 1, 4, 512, 512, 64, 1, ("packed", 40, 300), {}),
    (1, 1, 4, 384, 384, 128, 0, ("packed", 30, 120), {}),
    (1, 1, 4, 300, 420, 128, 0, ("packed", 20, 90), {}),  # T != S, ragged key block
    (1, 1, 2, 200, 456, 128, 2, ("packed", 20, 90), {}),  # end-aligned causal
    (1, 1, 4, 256, 256, 128, 1, ("scattered", (0, 1, 2)), {}),
    (1, 1, 8, 192, 192, 64, 0, ("scattered", (-7, 5, 2147483647)), {}),
    (1, 2, 4, 512, 512, 128, 1, ("packed", 30, 250), {"window": (100, -1)}),
    (1, 1, 4, 384, 384, 128, 1, ("packed", 30, 250), {"prefix": 40}),
    (1, 1, 4, 97, 97, 128, 1, ("packed", 5, 30), {}),  # a partial last query tile
]


def _id(c):
    B, K, G, T, S, H, causal, ids, kw = c
    return "B%dK%dG%dT%dS%dH%d_c%d_%s%s" % (B, K, G, T, S, H, causal, ids[0],
                                            "".join("_%s%s" % (k, v) for k, v in kw.items()))


def _ids(c):
    B, K, G, T, S, H, causal, ids, kw = c
    if ids[0] == "packed":
        q_seg = make_segment_ids(B, T, seed=T + 1, lo=ids[1], hi=ids[2])
        # end-aligned or T != S: the keys' ids are the queries' shifted to the end
        kv_seg = q_seg.clone() if T == S else make_segment_ids(B, S, seed=S + 3, lo=ids[1], hi=ids[2])
        return q_seg, kv_seg
    return _scattered_ids(B, T, T, ids[1]), _scattered_ids(B, S, S + 1, ids[1])


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_bwd_segments_vs_oracle_all_elements(case):
    B, K, G, T, S, H, causal, ids, kw = case
    q, k, v, do = make_qkv(B, K, G, T, S, H, seed=T * 3 + S, with_do=True)
    q_seg, kv_seg = _ids(case)
    qd, kd, vd, dod, qs, ks = to_dev(q, k, v, do, q_seg, kv_seg)
    o, lse = gqa.attn_fwd(qd, kd, vd, causal=causal, q_seg=qs, kv_seg=ks, **kw)
    dq, dk, dv = gqa.attn_bwd(qd, kd, vd, o, lse, dod, causal=causal, q_seg=qs, kv_seg=ks, **kw)
    torch.cuda.synchronize()
    ref = oracle.bwd(q, k, v, do, causal=causal, q_seg=q_seg, kv_seg=kv_seg, **kw)
    assert_close_all([("dQ", f32(dq), ref["dq"]), ("dK", f32(dk), ref["dk"]), ("dV", f32(dv), ref["dv"])])


def test_bwd_segments_at_the_query_cap_and_past_it():
    """T = 8192 takes the wave-pair kernel's id list at its capacity, T = 8256
    the general kernel; both against the oracle on sampled key rows (and the
    dQ rows of the same units)."""
    for T in (8192, 8256):
        B, K, G, H = 1, 1, 2, 64
        q, k, v, do = make_qkv(B, K, G, T, T, H, seed=T, with_do=True)
        q_seg = make_segment_ids(B, T, seed=5, lo=300, hi=3000)
        qd, kd, vd, dod, qs, ks = to_dev(q, k, v, do, q_seg, q_seg.clone())
        o, lse = gqa.attn_fwd(qd, kd, vd, causal=1, q_seg=qs, kv_seg=ks)
        dq, dk, dv = gqa.attn_bwd(qd, kd, vd, o, lse, dod, causal=1, q_seg=qs, kv_seg=ks)
        torch.cuda.synchronize()
        rng = np.random.default_rng(T)
        kvrows = np.unique(np.concatenate([rng.integers(0, T, 96), [0, 127, 128, T - 129, T - 1]]))
        qrows = np.unique(rng.integers(0, G * T, 96))
        ref = oracle.bwd(q, k, v, do, causal=1, q_seg=q_seg, kv_seg=q_seg.clone(), qrows=qrows, kvrows=kvrows)
        assert_close_all([("dQ", f32(dq).reshape(-1, H)[qrows], ref["dq"]),
                          ("dK", f32(dk).reshape(-1, H)[kvrows], ref["dk"]),
                          ("dV", f32(dv).reshape(-1, H)[kvrows], ref["dv"])])


def test_bwd_segments_deterministic():
    """The G-sum stays in the workgroup: two calls agree bit for bit."""
    B, K, G, T, H = 2, 2, 4, 1024, 128
    q, k, v, do = make_qkv(B, K, G, T, T, H, seed=3, with_do=True)
    q_seg = make_segment_ids(B, T, seed=9, lo=50, hi=400)
    qd, kd, vd, dod, qs, ks = to_dev(q, k, v, do, q_seg, q_seg.clone())
    o, lse = gqa.attn_fwd(qd, kd, vd, causal=1, q_seg=qs, kv_seg=ks)
    r1 = gqa.attn_bwd(qd, kd, vd, o, lse, dod, causal=1, q_seg=qs, kv_seg=ks)
    r2 = gqa.attn_bwd(qd, kd, vd, o, lse, dod, causal=1, q_seg=qs, kv_seg=ks)
    torch.cuda.synchronize()
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)


@pytest.mark.parametrize("causal", [0, 1])
def test_bwd_segments_query_block_without_keys(causal):
    """A whole query block (and a key block) whose ids appear on no key (no
    query): its list of tiles is empty, dQ of its rows is zero, and the
    other rows match the oracle."""
    B, K, G, T, H = 1, 2, 4, 512, 128
    q, k, v, do = make_qkv(B, K, G, T, T, H, seed=21, with_do=True)
    q_seg = make_segment_ids(B, T, seed=4, lo=60, hi=200)
    kv_seg = q_seg.clone()
    q_seg[:, 128:192] = 1000  # one 64-query block: no key has this id
    kv_seg[:, 320:448] = 2000  # one 128-key block: no query has it
    qd, kd, vd, dod, qs, ks = to_dev(q, k, v, do, q_seg, kv_seg)
    o, lse = gqa.attn_fwd(qd, kd, vd, causal=causal, q_seg=qs, kv_seg=ks)
    dq, dk, dv = gqa.attn_bwd(qd, kd, vd, o, lse, dod, causal=causal, q_seg=qs, kv_seg=ks)
    torch.cuda.synchronize()
    dq, dk, dv = f32(dq), f32(dk), f32(dv)
    assert np.all(dq[:, :, :, 128:192] == 0)
    assert np.all(dk[:, :, 320:448] == 0) and np.all(dv[:, :, 320:448] == 0)
    ref = oracle.bwd(q, k, v, do, causal=causal, q_seg=q_seg, kv_seg=kv_seg)
    assert_close_all([("dQ", dq, ref["dq"]), ("dK", dk, ref["dk"]), ("dV", dv, ref["dv"])])
