"""Helpers shared by the GPU parity tests (comparison metrics and row sampling)."""
import numpy as np
import torch

# Tolerances for O (bf16 output vs fp64 oracle on the same bf16 inputs):
# max-abs 2e-2 and relative L2 5e-3 over the compared elements.
O_MAX_ABS = 2e-2
O_REL_L2 = 5e-3
# lse is fp32 from fp32-accumulated bf16 products; one rounding of the
# logits and of ln(l) keeps it well inside 1e-3.
LSE_MAX_ABS = 1e-3


def rel_l2(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    return np.linalg.norm((x - ref).ravel()) / (den if den > 0 else 1.0)


def max_abs(x, ref):
    return float(np.max(np.abs(np.asarray(x, dtype=np.float64) - np.asarray(ref, dtype=np.float64))))


def assert_close_o(x, ref, what="O"):
    ma, rl = max_abs(x, ref), rel_l2(x, ref)
    assert ma <= O_MAX_ABS and rl <= O_REL_L2, "%s: max-abs %.3e (<= %.0e), rel-L2 %.3e (<= %.0e)" % (
        what, ma, O_MAX_ABS, rl, O_REL_L2)
    return ma, rl


def assert_close_all(pairs):
    """Check several (name, got, ref) triples and report every failure at once."""
    errs = []
    for name, x, ref in pairs:
        ma, rl = max_abs(x, ref), rel_l2(x, ref)
        if not (ma <= O_MAX_ABS and rl <= O_REL_L2):
            errs.append("%s: max-abs %.3e rel-L2 %.3e" % (name, ma, rl))
    assert not errs, "; ".join(errs)


def assert_close_lse(x, ref, what="lse"):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.array_equal(np.isneginf(x), np.isneginf(ref)), what + ": -inf pattern differs"
    fin = np.isfinite(ref)
    if fin.any():
        ma = max_abs(x[fin], ref[fin])
        assert ma <= LSE_MAX_ABS, "%s: max-abs %.3e" % (what, ma)


def sample_rows(B, K, G, T, n, seed):
    """Flat row indices into [B,K,G,T]: first and last query of every (b,k,g)
    head plus n random rows."""
    rng = np.random.default_rng(seed)
    heads = np.arange(B * K * G) * T
    rows = np.concatenate([heads, heads + T - 1, rng.integers(0, B * K * G * T, size=n)])
    return np.unique(rows)


def to_dev(*ts):
    return [None if t is None else t.cuda() for t in ts]


def f32(t):
    return t.detach().float().cpu().numpy()
