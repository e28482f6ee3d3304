"""The Python binding refuses every malformed argument before anything is
launched: device, dtype, shape and contiguity of every tensor (segment ids,
dO, v, a caller workspace) for the forward and the backward. Outputs passed
in keep their contents, which shows that no kernel ran."""
import pytest
import torch

import grouped_query_attention_flash_amd as gqa
from parity_util import to_dev
from workloads import make_qkv, make_segment_ids

pytestmark = pytest.mark.gpu

B, K, G, T, S, H = 1, 2, 4, 128, 192, 128


@pytest.fixture(scope="module")
def inputs():
    q, k, v, do = to_dev(*make_qkv(B, K, G, T, S, H, seed=151, with_do=True))
    qs = make_segment_ids(B, T, seed=1, lo=10, hi=40).cuda()
    ks = make_segment_ids(B, S, seed=2, lo=10, hi=40).cuda()
    o, lse = gqa.attn_fwd(q, k, v, causal=True, q_seg=qs, kv_seg=ks)
    torch.cuda.synchronize()
    return dict(q=q, k=k, v=v, do=do, qs=qs, ks=ks, o=o, lse=lse)


def _sentinels(d):
    dq = torch.full(d["q"].shape, 7.0, dtype=torch.float32, device="cuda")
    dk = torch.full(d["k"].shape, 7.0, dtype=torch.float32, device="cuda")
    dv = torch.full(d["k"].shape, 7.0, dtype=torch.float32, device="cuda")
    return dq, dk, dv


BWD_BAD = [
    ("q_seg on the host", lambda d: dict(q_seg=d["qs"].cpu())),
    ("kv_seg on the host", lambda d: dict(kv_seg=d["ks"].cpu())),
    ("q_seg int64", lambda d: dict(q_seg=d["qs"].long())),
    ("q_seg wrong shape", lambda d: dict(q_seg=d["ks"])),
    ("kv_seg wrong shape", lambda d: dict(kv_seg=d["qs"])),
    ("only q_seg", lambda d: dict(kv_seg=None)),
    ("v wrong shape", lambda d: dict(v=d["v"][:, :, :S - 1].contiguous())),
    ("dO wrong shape", lambda d: dict(do=d["do"][:, :, :, :T - 1].contiguous())),
    ("dO fp32", lambda d: dict(do=d["do"].float())),
    ("dO on the host", lambda d: dict(do=d["do"].cpu())),
    ("dO not contiguous", lambda d: dict(do=d["do"].transpose(3, 4).contiguous().transpose(3, 4))),
    ("workspace on the host", lambda d: dict(workspace=torch.empty(1 << 20, dtype=torch.uint8))),
    ("workspace fp32", lambda d: dict(workspace=torch.empty(1 << 18, dtype=torch.float32, device="cuda"))),
    ("workspace too small", lambda d: dict(workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))),
    ("lse wrong shape", lambda d: dict(lse=d["lse"][..., :T - 1].contiguous())),
    ("causal mode 3", lambda d: dict(causal=3)),
    ("negative prefix", lambda d: dict(prefix=-2)),
    ("window side -2", lambda d: dict(window=(-2, 0))),
]


@pytest.mark.parametrize("name,bad", BWD_BAD, ids=[b[0] for b in BWD_BAD])
def test_bwd_refuses_before_launch(inputs, name, bad):
    d = inputs
    dq, dk, dv = _sentinels(d)
    kw = dict(q_seg=d["qs"], kv_seg=d["ks"], causal=True, dq=dq, dk=dk, dv=dv)
    args = dict(q=d["q"], k=d["k"], v=d["v"], o=d["o"], lse=d["lse"], do=d["do"])
    over = bad(d)
    for key in list(over):
        if key in args:
            args[key] = over.pop(key)
    kw.update(over)
    with pytest.raises(ValueError):
        gqa.attn_bwd(args["q"], args["k"], args["v"], args["o"], args["lse"], args["do"], **kw)
    torch.cuda.synchronize()
    assert bool((dq == 7.0).all() and (dk == 7.0).all() and (dv == 7.0).all()), name


FWD_BAD = [
    ("q_seg on the host", lambda d: dict(q_seg=d["qs"].cpu())),
    ("kv_seg int16", lambda d: dict(kv_seg=d["ks"].short())),
    ("kv_seg wrong shape", lambda d: dict(kv_seg=d["qs"])),
    ("v wrong shape", lambda d: dict(v=d["v"][:, :, :S - 1].contiguous())),
    ("k on the host", lambda d: dict(k=d["k"].cpu())),
    ("workspace on the host", lambda d: dict(split_kv=True, workspace=torch.empty(1 << 20, dtype=torch.uint8))),
    ("workspace int32", lambda d: dict(split_kv=True,
                                       workspace=torch.empty(1 << 18, dtype=torch.int32, device="cuda"))),
    ("lse on the host", lambda d: dict(lse=torch.empty(B, K, G, T))),
    ("causal mode -1", lambda d: dict(causal=-1)),
    ("prefix negative", lambda d: dict(prefix=-1)),
]


@pytest.mark.parametrize("name,bad", FWD_BAD, ids=[b[0] for b in FWD_BAD])
def test_fwd_refuses_before_launch(inputs, name, bad):
    d = inputs
    out = torch.full_like(d["q"], 3.0)
    args = dict(q=d["q"], k=d["k"], v=d["v"])
    kw = dict(q_seg=d["qs"], kv_seg=d["ks"], causal=True, out=out)
    over = bad(d)
    for key in list(over):
        if key in args:
            args[key] = over.pop(key)
    kw.update(over)
    with pytest.raises(ValueError):
        gqa.attn_fwd(args["q"], args["k"], args["v"], **kw)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()), name
