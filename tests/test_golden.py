"""Hand-derived worked examples (tests/golden/hand_examples.json) against the oracle."""
import json
import math
import os

import numpy as np
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _eval(expr):
    return eval(expr, {"__builtins__": {}}, {"e": math.e, "exp": math.exp, "log": math.log})


def test_hand_examples():
    with open(os.path.join(HERE, "golden", "hand_examples.json")) as f:
        cases = json.load(f)
    for c in cases:
        B, K, G, T, S, H = (c[x] for x in "BKGTSH")
        q = torch.tensor(c["q"], dtype=torch.float32).reshape(B, K, G, T, H).to(torch.bfloat16)
        k = torch.tensor(c["k"], dtype=torch.float32).reshape(B, K, S, H).to(torch.bfloat16)
        v = torch.tensor(c["v"], dtype=torch.float32).reshape(B, K, S, H).to(torch.bfloat16)
        for name, t in (("q", q), ("k", k), ("v", v)):  # inputs must be exact in bf16
            assert torch.equal(t.float().flatten(), torch.tensor(c[name], dtype=torch.float32)), (c["name"], name)
        kw = {}
        if "q_seg" in c:
            kw = dict(q_seg=torch.tensor([c["q_seg"]], dtype=torch.int32),
                      kv_seg=torch.tensor([c["kv_seg"]], dtype=torch.int32))
        o, lse = oracle.fwd(q, k, v, causal=c["causal"], **kw)
        np.testing.assert_allclose(o.flatten(), [_eval(x) for x in c["o"]], atol=1e-15, err_msg=c["name"])
        np.testing.assert_allclose(lse.flatten(), [_eval(x) for x in c["lse"]], atol=1e-15, err_msg=c["name"])
