"""CPU oracle for masked grouped-query softmax attention (fp64).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU
baseline leg import this package; the product path (the HIP library and its
Python binding) never does, and shares no code with it.

``fwd`` and ``bwd`` call the plain fp64 C definition in ``gqa_oracle.c``.
``fwd(..., precision="f32")`` calls the same source built with float
accumulation (``libgqa_oracle_f32.so``): a timed CPU baseline only, checked
against the fp64 build, never a parity reference.
``online.chunked_fwd`` is a separate numpy model of the chunked
online-softmax recurrence, used only to cross-check the plain definition.

Inputs are torch bf16 CPU tensors (or numpy uint16 bit patterns) in the
layout q/dO [B,K,G,T,H], k/v [B,K,S,H], segment ids int32 [B,T]/[B,S],
explicit mask bool [B,T,S].
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gqa_oracle.c")
_LIB = os.path.join(_HERE, "libgqa_oracle.so")
_LIB_F32 = os.path.join(_HERE, "libgqa_oracle_f32.so")
_libs = {}


def _build_one(path, defines, force):
    if force or not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
        tmp = path + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", *defines, "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, path)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP): the fp64 build and the
    float-accumulation build of the same source. Returns the fp64 path."""
    _build_one(_LIB, [], force)
    _build_one(_LIB_F32, ["-DORACLE_ACC_FLOAT"], force)
    return _LIB


def _load(precision="f64"):
    if precision not in _libs:
        path = {"f64": _LIB, "f32": _LIB_F32}[precision]
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_fwd_rows.restype = ctypes.c_int
        lib.oracle_fwd_rows.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I64, I64, ctypes.c_int,
                                        I64, I64, I64, I64, P, P, P]
        lib.oracle_bwd_rows.restype = ctypes.c_int
        lib.oracle_bwd_rows.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I64, ctypes.c_int,
                                        I64, I64, I64, I64, P, P, P, I64, P, P, P]
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        _libs[precision] = lib
    return _libs[precision]


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def _bits(x):
    """bf16 tensor / uint16 array -> contiguous numpy uint16 bit patterns."""
    if isinstance(x, np.ndarray):
        assert x.dtype == np.uint16
        return np.ascontiguousarray(x)
    import torch
    assert x.dtype == torch.bfloat16, x.dtype
    return np.ascontiguousarray(x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def _i32(x):
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        return np.ascontiguousarray(x, dtype=np.int32)
    return np.ascontiguousarray(x.detach().cpu().numpy().astype(np.int32))


def _u8(x):
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        return np.ascontiguousarray(x.astype(np.uint8))
    return np.ascontiguousarray(x.detach().cpu().numpy().astype(np.uint8))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _rows(rows):
    if rows is None:
        return None
    return np.ascontiguousarray(np.asarray(rows, dtype=np.int64))


def _window(window):
    if window is None:
        return -1, -1
    wl, wr = int(window[0]), int(window[1])
    assert wl >= -1 and wr >= -1
    return wl, wr


def _causal(causal):
    """0 none, 1 top-left (s <= t), 2 end-aligned (s <= t + S - T)."""
    if isinstance(causal, str):
        return {"none": 0, "top_left": 1, "end": 2}[causal]
    c = int(causal)
    assert c in (0, 1, 2), causal
    return c


def fwd(q, k, v, *, causal=False, q_seg=None, kv_seg=None, mask=None, rows=None, window=None, prefix=0,
        precision="f64"):
    """Plain fp64 attention. Returns (O, lse) as float64 numpy arrays.

    rows=None: O has q's shape and lse q's shape minus H.
    rows given (flat indices into [B,K,G,T]): O is [len(rows), H], lse [len(rows)].
    causal: False/0, True/1 (s <= t), 2 or "end" (s <= t + S - T).
    window=(wl, wr): key s visible to query t only if t - wl <= s <= t + wr
    (a side of -1 is unbounded). prefix=p: keys s < p are visible to every
    query whatever the causal rule and window say (segments still apply).
    precision="f32" runs the float-accumulation build (timing only).
    """
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    B, K, G, T, H = qb.shape
    S = kb.shape[2]
    assert kb.shape == (B, K, S, H) and vb.shape == kb.shape
    qs, ks, mk = _i32(q_seg), _i32(kv_seg), _u8(mask)
    if mk is not None:
        assert mk.shape == (B, T, S)
    r = _rows(rows)
    n = B * K * G * T if r is None else len(r)
    o = np.empty((n, H), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = _load(precision).oracle_fwd_rows(_ptr(qb), _ptr(kb), _ptr(vb), _ptr(qs), _ptr(ks), _ptr(mk),
                                 B, K, G, T, S, H, _causal(causal), *_window(window), int(prefix), n, _ptr(r),
                                 _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_fwd_rows failed with code %d" % rc)
    if r is None:
        return o.reshape(B, K, G, T, H), lse.reshape(B, K, G, T)
    return o, lse


def bwd(q, k, v, do, *, causal=False, q_seg=None, kv_seg=None, mask=None, qrows=None, kvrows=None,
        want_dq=True, want_dkv=True, window=None, prefix=0):
    """Plain fp64 gradients of sum(O * dO). Returns dict with dq, dk, dv, D.

    Full tensors when the row lists are None, else [n, H] arrays for the
    listed rows (qrows index [B,K,G,T], kvrows index [B,K,S])."""
    qb, kb, vb, db = _bits(q), _bits(k), _bits(v), _bits(do)
    B, K, G, T, H = qb.shape
    S = kb.shape[2]
    assert db.shape == qb.shape
    qs, ks, mk = _i32(q_seg), _i32(kv_seg), _u8(mask)
    qr, kr = _rows(qrows), _rows(kvrows)
    nq = (B * K * G * T if qr is None else len(qr)) if want_dq else 0
    nkv = (B * K * S if kr is None else len(kr)) if want_dkv else 0
    if not want_dq:
        qr = np.zeros(0, dtype=np.int64)
    if not want_dkv:
        kr = np.zeros(0, dtype=np.int64)
    dq = np.empty((max(nq, 1), H), dtype=np.float64)
    dd = np.empty((max(nq, 1),), dtype=np.float64)
    dk = np.empty((max(nkv, 1), H), dtype=np.float64)
    dv = np.empty((max(nkv, 1), H), dtype=np.float64)
    rc = _load().oracle_bwd_rows(_ptr(qb), _ptr(kb), _ptr(vb), _ptr(db), _ptr(qs), _ptr(ks), _ptr(mk),
                                 B, K, G, T, S, H, _causal(causal), *_window(window), int(prefix),
                                 nq, _ptr(qr), _ptr(dq) if nq else None, _ptr(dd) if nq else None,
                                 nkv, _ptr(kr), _ptr(dk) if nkv else None, _ptr(dv) if nkv else None)
    if rc != 0:
        raise ValueError("oracle_bwd_rows failed with code %d" % rc)
    out = {}
    if want_dq:
        dq, dd = dq[:nq], dd[:nq]
        if qrows is None:
            dq, dd = dq.reshape(B, K, G, T, H), dd.reshape(B, K, G, T)
        out["dq"], out["D"] = dq, dd
    if want_dkv:
        dk, dv = dk[:nkv], dv[:nkv]
        if kvrows is None:
            dk, dv = dk.reshape(B, K, S, H), dv.reshape(B, K, S, H)
        out["dk"], out["dv"] = dk, dv
    return out


if __name__ == "__main__":
    print(build(force=True), file=sys.stderr)
