"""The chunked online-softmax recurrence in numpy fp64 (test infrastructure).

TEST INFRASTRUCTURE ONLY. This is a second, independent model of what the
fused kernel computes, written from the recurrence on danielwatson6.github.io/fa
("Chunked attention", the numerically stable scan, and "Optimizing the
kernel", the fused two-axis version): the keys are visited in chunks; a
running row maximum m, a running denominator and an fp32-style output carry
are rescaled by exp(m_old - m_new) whenever the maximum grows, and the carry
is divided by the denominator at the end. Tests check that it agrees with the
plain definition in ``gqa_oracle.c`` to rounding, for any chunk size, which
pins the claim that the recurrence is an exact re-association of softmax.

Masked logits are set to -inf. A chunk in which a row has seen no visible key
yet would give exp(-inf - (-inf)); the model treats that row's reference
maximum as 0 for the exponentials, so its carries stay exactly zero (the page
does not mask and so never meets this case).

``round_p_bf16`` mimics the page's cast of the weights to bf16 before the
second matmul; it is a diagnostic and is off for parity.
"""
from __future__ import annotations

import numpy as np


def _bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _round_bf16(x: np.ndarray) -> np.ndarray:
    f = x.astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def chunked_fwd(q_bits, k_bits, v_bits, *, bkv: int, causal=False, q_seg=None, kv_seg=None,
                round_p_bf16=False):
    """Chunked online softmax over key chunks of size bkv (last chunk may be short).

    q_bits [B,K,G,T,H], k_bits/v_bits [B,K,S,H] as uint16 bf16 patterns.
    Returns (O [B,K,G,T,H], lse [B,K,G,T]) in float64."""
    q = _bf16_bits_to_f64(q_bits)
    k = _bf16_bits_to_f64(k_bits)
    v = _bf16_bits_to_f64(v_bits)
    B, K, G, T, H = q.shape
    S = k.shape[2]
    o = np.zeros((B, K, G, T, H))
    denom = np.zeros((B, K, G, T))
    m = np.full((B, K, G, T), -np.inf)
    t_idx = np.arange(T)[:, None]
    for s0 in range(0, S, bkv):
        s1 = min(S, s0 + bkv)
        kb, vb = k[:, :, s0:s1], v[:, :, s0:s1]
        lb = np.einsum("bkgth,bksh->bkgts", q, kb)
        vis = np.ones((B, 1, 1, T, s1 - s0), dtype=bool)
        if causal:
            vis &= (np.arange(s0, s1)[None, :] <= t_idx)[None, None, None]
        if q_seg is not None:
            qs = np.asarray(q_seg)[:, :, None]
            ks = np.asarray(kv_seg)[:, None, s0:s1]
            vis &= (qs == ks)[:, None, None]
        lb = np.where(vis, lb, -np.inf)
        m_new = np.maximum(m, lb.max(axis=-1))
        ref = np.where(np.isneginf(m_new), 0.0, m_new)
        corr = np.exp(m - ref)
        w = np.exp(lb - ref[..., None])
        denom = denom * corr + w.sum(axis=-1)
        wp = _round_bf16(w) if round_p_bf16 else w
        o = o * corr[..., None] + np.einsum("bkgts,bksh->bkgth", wp, vb)
        m = m_new
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(denom[..., None] > 0, o / np.where(denom > 0, denom, 1.0)[..., None], 0.0)
        lse = np.where(denom > 0, m + np.log(np.where(denom > 0, denom, 1.0)), -np.inf)
    return out, lse
