"""Python binding of libgqa_attn.so, the fused grouped-query flash-attention
library for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/gqa_attn.h. PyTorch provides
device memory and the current stream; there is no CPU or PyTorch fallback --
if the library is missing or fails, these functions raise.

Layouts: q, o, dO [B, K, G, T, H] bf16 (q pre-multiplied by H^-1/2);
k, v [B, K, S, H] bf16; lse [B, K, G, T] fp32; q_seg [B, T] and
kv_seg [B, S] int32; gradients fp32 in the layouts of their inputs.

Masks (all lazy): causal=False/0 (none), True/1 or "top_left" (s <= t),
2 or "end" (s <= t + S - T, end-aligned); window=(left, right) with -1 for
an unbounded side; prefix=p makes keys s < p visible to every query.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgqa_attn.so")

GQA_ATTN_OK = 0
GQA_ATTN_ERR_NULL = 1
GQA_ATTN_ERR_SHAPE = 2
GQA_ATTN_ERR_HEADDIM = 3
GQA_ATTN_ERR_ALIGN = 4
GQA_ATTN_ERR_SEGMENTS = 5
GQA_ATTN_ERR_WORKSPACE = 6
GQA_ATTN_ERR_HIP = 7
GQA_ATTN_ERR_MASK = 8
GQA_ATTN_ERR_TUNING = 9

CAUSAL_NONE, CAUSAL_TOP_LEFT, CAUSAL_END = 0, 1, 2

EXPORTED_SYMBOLS = (
    "attn_fwd", "attn_check_fwd", "attn_fwd_ws", "attn_check_fwd_ws", "attn_fwd_workspace_bytes",
    "attn_fwd_split_count", "attn_fwd_local", "attn_check_fwd_local", "attn_fwd_mask", "attn_check_fwd_mask",
    "attn_bwd_workspace_bytes", "attn_bwd", "attn_check_bwd", "attn_bwd_local", "attn_check_bwd_local",
    "attn_bwd_mask", "attn_check_bwd_mask", "attn_fwd_noalloc", "attn_fwd_tuned", "attn_fwd_tuned_workspace_bytes",
    "attn_fwd_tuning", "attn_fwd_head_masks", "attn_check_fwd_head_masks", "attn_bwd_head_masks",
    "attn_check_bwd_head_masks", "attn_strerror", "attn_last_hip_error",
)

_lib = None


class GqaAttnError(ValueError):
    """A nonzero return code of the C library."""

    def __init__(self, code: int, where: str):
        self.code = code
        msg = attn_strerror(code)
        if code == GQA_ATTN_ERR_HIP:
            msg += " (hipError %d)" % attn_last_hip_error()
        super().__init__("%s: %s [code %d]" % (where, msg, code))


def load_library():
    """Load libgqa_attn.so (built by grouped_query_attention_flash_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libgqa_attn.so is not built (%s); run `python -m grouped_query_attention_flash_amd.build`"
                           % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.attn_fwd.restype = I
    lib.attn_fwd.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, P]
    lib.attn_check_fwd.restype = I
    lib.attn_check_fwd.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I]
    lib.attn_fwd_ws.restype = I
    lib.attn_fwd_ws.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, SZ, P]
    lib.attn_check_fwd_ws.restype = I
    lib.attn_check_fwd_ws.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, SZ]
    lib.attn_fwd_local.restype = I
    lib.attn_fwd_local.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, P, SZ, P]
    lib.attn_check_fwd_local.restype = I
    lib.attn_check_fwd_local.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, P, SZ]
    lib.attn_fwd_mask.restype = I
    lib.attn_fwd_mask.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, P, SZ, P]
    lib.attn_check_fwd_mask.restype = I
    lib.attn_check_fwd_mask.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, P, SZ]
    lib.attn_bwd_local.restype = I
    lib.attn_bwd_local.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, P, SZ, P]
    lib.attn_check_bwd_local.restype = I
    lib.attn_check_bwd_local.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, P, SZ]
    lib.attn_bwd_mask.restype = I
    lib.attn_bwd_mask.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, P, SZ, P]
    lib.attn_check_bwd_mask.restype = I
    lib.attn_check_bwd_mask.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, P, SZ]
    lib.attn_fwd_tuned.restype = I
    lib.attn_fwd_tuned.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, I, I, P, SZ, P]
    lib.attn_fwd_tuned_workspace_bytes.restype = SZ
    lib.attn_fwd_tuned_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.attn_fwd_tuning.restype = I
    lib.attn_fwd_tuning.argtypes = [I, I, I, I, I, I, I, I, I, I, I, P, P]
    lib.attn_fwd_noalloc.restype = I
    lib.attn_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, P]
    lib.attn_fwd_workspace_bytes.restype = SZ
    lib.attn_fwd_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.attn_fwd_split_count.restype = I
    lib.attn_fwd_split_count.argtypes = [I, I, I, I, I, I]
    lib.attn_bwd_workspace_bytes.restype = SZ
    lib.attn_bwd_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.attn_bwd.restype = I
    lib.attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, SZ, P]
    lib.attn_check_bwd.restype = I
    lib.attn_check_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, SZ]
    lib.attn_fwd_head_masks.restype = I
    lib.attn_fwd_head_masks.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, P]
    lib.attn_check_fwd_head_masks.restype = I
    lib.attn_check_fwd_head_masks.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, P]
    lib.attn_bwd_head_masks.restype = I
    lib.attn_bwd_head_masks.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, P, SZ, P]
    lib.attn_check_bwd_head_masks.restype = I
    lib.attn_check_bwd_head_masks.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, P, SZ]
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_strerror.argtypes = [I]
    lib.attn_last_hip_error.restype = I
    lib.attn_last_hip_error.argtypes = []
    _lib = lib
    return lib


def attn_strerror(code: int) -> str:
    return load_library().attn_strerror(int(code)).decode()


def attn_last_hip_error() -> int:
    return int(load_library().attn_last_hip_error())


def attn_bwd_workspace_bytes(B: int, K: int, G: int, T: int, S: int, H: int) -> int:
    return int(load_library().attn_bwd_workspace_bytes(B, K, G, T, S, H))


def attn_fwd_workspace_bytes(B: int, K: int, G: int, T: int, S: int, H: int) -> int:
    return int(load_library().attn_fwd_workspace_bytes(B, K, G, T, S, H))


def attn_fwd_split_count(B: int, K: int, G: int, T: int, S: int, H: int) -> int:
    return int(load_library().attn_fwd_split_count(B, K, G, T, S, H))


def attn_fwd_tuning(B: int, K: int, G: int, T: int, S: int, H: int, causal=False, window=None, prefix: int = 0,
                    segments: bool = False) -> Tuple[int, int]:
    """The tuning table's (load_placement, split_target) for a call (host only)."""
    lp, st = ctypes.c_int(-2), ctypes.c_int(-2)
    wl, wr = (-1, -1) if window is None else (int(window[0]), int(window[1]))
    rc = load_library().attn_fwd_tuning(B, K, G, T, S, H, causal_mode(causal), wl, wr, int(prefix), int(bool(segments)),
                                        ctypes.byref(lp), ctypes.byref(st))
    if rc != GQA_ATTN_OK:
        raise GqaAttnError(rc, "attn_fwd_tuning")
    return lp.value, st.value


def attn_fwd_tuned_workspace_bytes(B: int, K: int, G: int, T: int, S: int, H: int, split_target: int = -1) -> int:
    return int(load_library().attn_fwd_tuned_workspace_bytes(B, K, G, T, S, H, int(split_target)))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dims(q: torch.Tensor, k: torch.Tensor):
    if q.dim() != 5 or k.dim() != 4:
        raise ValueError("q must be [B,K,G,T,H] and k, v [B,K,S,H]")
    B, K, G, T, H = q.shape
    if k.shape[0] != B or k.shape[1] != K or k.shape[3] != H:
        raise ValueError("k shape %s does not match q shape %s" % (tuple(k.shape), tuple(q.shape)))
    return B, K, G, T, k.shape[2], H


def _check_tensor(name, t, dtype, shape=None, device=None):
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if device is not None and t.device != device:
        raise ValueError("%s must be on %s, got %s" % (name, device, t.device))
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def causal_mode(causal) -> int:
    """The C ABI's causal argument: False/0 none, True/1/"top_left" s <= t,
    2/"end" s <= t + S - T (end-aligned)."""
    if isinstance(causal, str):
        modes = {"none": CAUSAL_NONE, "top_left": CAUSAL_TOP_LEFT, "end": CAUSAL_END}
        if causal not in modes:
            raise ValueError("causal must be one of %s, got %r" % (sorted(modes), causal))
        return modes[causal]
    c = int(causal)
    if c not in (CAUSAL_NONE, CAUSAL_TOP_LEFT, CAUSAL_END):
        raise GqaAttnError(GQA_ATTN_ERR_MASK, "causal=%r" % (causal,))
    return c


def _check_segments(q_seg, kv_seg, B, T, S, device, where):
    if (q_seg is None) != (kv_seg is None):
        raise GqaAttnError(GQA_ATTN_ERR_SEGMENTS, where)
    if q_seg is not None:
        _check_tensor("q_seg", q_seg, torch.int32, (B, T), device)
        _check_tensor("kv_seg", kv_seg, torch.int32, (B, S), device)


def _check_workspace(workspace, device):
    if workspace is not None:
        _check_tensor("workspace", workspace, torch.uint8, None, device)
        if workspace.dim() != 1:
            raise ValueError("workspace must be a 1-D uint8 tensor")


def _check_head_mask(head_mask, K, G, device):
    _check_tensor("head_mask", head_mask, torch.int32, (K, G, 3), device)


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal=False,
             q_seg: Optional[torch.Tensor] = None, kv_seg: Optional[torch.Tensor] = None,
             out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
             want_lse: bool = True, split_kv: bool = False,
             workspace: Optional[torch.Tensor] = None,
             window: Optional[Tuple[int, int]] = None,
             prefix: int = 0, head_mask: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Forward pass on the current stream. Returns (o, lse).

    causal: see causal_mode(). split_kv=True calls attn_fwd_ws, which splits
    the key range across workgroups for shapes that would leave the GPU idle
    (decoding); the workspace (uint8, at least attn_fwd_workspace_bytes) is
    allocated when not given. window=(left, right) and / or prefix=p call
    attn_fwd_mask: key s is visible to query t when s < p or t - left <= s <=
    t + right (-1: unbounded side) and the causal rule holds; it splits like
    split_kv. head_mask (int32 [K, G, 3] on the device: window left, window
    right, prefix per query head) calls attn_fwd_head_masks instead: each
    query head takes its own window and prefix; it excludes window, prefix
    and split_kv."""
    B, K, G, T, S, H = _dims(q, k)
    dev = q.device
    _check_tensor("q", q, torch.bfloat16)
    _check_tensor("k", k, torch.bfloat16, None, dev)
    _check_tensor("v", v, torch.bfloat16, k.shape, dev)
    cm = causal_mode(causal)
    _check_segments(q_seg, kv_seg, B, T, S, dev, "attn_fwd")
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, torch.bfloat16, q.shape, dev)
    if lse is None and want_lse:
        lse = torch.empty(B, K, G, T, dtype=torch.float32, device=dev)
    if lse is not None:
        _check_tensor("lse", lse, torch.float32, (B, K, G, T), dev)
    if head_mask is not None:
        if window is not None or prefix != 0 or split_kv:
            raise ValueError("head_mask excludes window, prefix and split_kv")
        _check_head_mask(head_mask, K, G, dev)
        rc = load_library().attn_fwd_head_masks(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(q_seg),
                                                _ptr(kv_seg), B, K, G, T, S, H, cm, _ptr(head_mask),
                                                _stream_handle(dev))
        if rc != GQA_ATTN_OK:
            raise GqaAttnError(rc, "attn_fwd_head_masks")
        return out, lse
    masked = window is not None or prefix != 0
    if masked or split_kv:
        wsb = attn_fwd_workspace_bytes(B, K, G, T, S, H)
        if workspace is None and wsb > 0:
            workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
        _check_workspace(workspace, dev)
    wsp, wsn = _ptr(workspace), 0 if workspace is None else workspace.numel()
    if masked:
        wl, wr = (-1, -1) if window is None else (int(window[0]), int(window[1]))
        rc = load_library().attn_fwd_mask(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(q_seg),
                                          _ptr(kv_seg), B, K, G, T, S, H, cm, wl, wr, int(prefix), wsp, wsn,
                                          _stream_handle(dev))
        if rc != GQA_ATTN_OK:
            raise GqaAttnError(rc, "attn_fwd_mask")
        return out, lse
    if split_kv:
        rc = load_library().attn_fwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(q_seg), _ptr(kv_seg),
                                        B, K, G, T, S, H, cm, wsp, wsn, _stream_handle(dev))
        if rc != GQA_ATTN_OK:
            raise GqaAttnError(rc, "attn_fwd_ws")
        return out, lse
    rc = load_library().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(q_seg), _ptr(kv_seg),
                                 B, K, G, T, S, H, cm, _stream_handle(dev))
    if rc != GQA_ATTN_OK:
        raise GqaAttnError(rc, "attn_fwd")
    return out, lse


def attn_fwd_tuned(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, load_placement: int = -1,
                   split_target: int = -1, causal=False, q_seg: Optional[torch.Tensor] = None,
                   kv_seg: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, window: Optional[Tuple[int, int]] = None, prefix: int = 0,
                   workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """attn_fwd_mask with an explicit schedule (attn_fwd_tuned): load_placement
    (0, 1, 2) and split_target (0 .. 2^20); -1 takes the tuning table's choice."""
    B, K, G, T, S, H = _dims(q, k)
    dev = q.device
    _check_tensor("q", q, torch.bfloat16)
    _check_tensor("k", k, torch.bfloat16, None, dev)
    _check_tensor("v", v, torch.bfloat16, k.shape, dev)
    cm = causal_mode(causal)
    _check_segments(q_seg, kv_seg, B, T, S, dev, "attn_fwd_tuned")
    out = torch.empty_like(q) if out is None else out
    _check_tensor("out", out, torch.bfloat16, q.shape, dev)
    lse = torch.empty(B, K, G, T, dtype=torch.float32, device=dev) if lse is None else lse
    _check_tensor("lse", lse, torch.float32, (B, K, G, T), dev)
    wsb = attn_fwd_tuned_workspace_bytes(B, K, G, T, S, H, split_target)
    if workspace is None and wsb > 0:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    _check_workspace(workspace, dev)
    wl, wr = (-1, -1) if window is None else (int(window[0]), int(window[1]))
    rc = load_library().attn_fwd_tuned(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(q_seg), _ptr(kv_seg),
                                       B, K, G, T, S, H, cm, wl, wr, int(prefix), int(load_placement),
                                       int(split_target), _ptr(workspace),
                                       0 if workspace is None else workspace.numel(), _stream_handle(dev))
    if rc != GQA_ATTN_OK:
        raise GqaAttnError(rc, "attn_fwd_tuned")
    return out, lse


def attn_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                     lse: Optional[torch.Tensor] = None, *, causal=False,
                     q_seg: Optional[torch.Tensor] = None, kv_seg: Optional[torch.Tensor] = None,
                     window: Optional[Tuple[int, int]] = None, prefix: int = 0) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """attn_fwd_mask without a workspace (attn_fwd_noalloc): the library keeps
    the split-KV partials in its own static device array (16 MiB per GPU), so
    neither this call nor the library allocates device memory; the caller
    passes `out` (and `lse`, or None). Calls that overlap on one GPU share
    that array and must not run concurrently."""
    B, K, G, T, S, H = _dims(q, k)
    dev = q.device
    _check_tensor("q", q, torch.bfloat16)
    _check_tensor("k", k, torch.bfloat16, None, dev)
    _check_tensor("v", v, torch.bfloat16, k.shape, dev)
    _check_tensor("out", out, torch.bfloat16, q.shape, dev)
    if lse is not None:
        _check_tensor("lse", lse, torch.float32, (B, K, G, T), dev)
    cm = causal_mode(causal)
    _check_segments(q_seg, kv_seg, B, T, S, dev, "attn_fwd_noalloc")
    wl, wr = (-1, -1) if window is None else (int(window[0]), int(window[1]))
    rc = load_library().attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(q_seg), _ptr(kv_seg),
                                         B, K, G, T, S, H, cm, wl, wr, int(prefix), _stream_handle(dev))
    if rc != GQA_ATTN_OK:
        raise GqaAttnError(rc, "attn_fwd_noalloc")
    return out, lse


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: Optional[torch.Tensor], lse: torch.Tensor,
             do: torch.Tensor, *, causal=False, q_seg: Optional[torch.Tensor] = None,
             kv_seg: Optional[torch.Tensor] = None, dq: Optional[torch.Tensor] = None,
             dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None, window: Optional[Tuple[int, int]] = None,
             prefix: int = 0, head_mask: Optional[torch.Tensor] = None):
    """Backward pass on the current stream. Returns (dq, dk, dv) in fp32.

    `o` (the forward output) may be None: the library does not read it.
    window / prefix call attn_bwd_mask with the forward's mask; head_mask
    (as in attn_fwd) calls attn_bwd_head_masks. Every tensor
    is checked (device, dtype, shape, contiguity) before anything is
    launched."""
    B, K, G, T, S, H = _dims(q, k)
    dev = q.device
    _check_tensor("q", q, torch.bfloat16)
    _check_tensor("k", k, torch.bfloat16, None, dev)
    _check_tensor("v", v, torch.bfloat16, k.shape, dev)
    _check_tensor("do", do, torch.bfloat16, q.shape, dev)
    if o is not None:
        _check_tensor("o", o, torch.bfloat16, q.shape, dev)
    _check_tensor("lse", lse, torch.float32, (B, K, G, T), dev)
    cm = causal_mode(causal)
    _check_segments(q_seg, kv_seg, B, T, S, dev, "attn_bwd")
    dq = torch.empty(q.shape, dtype=torch.float32, device=dev) if dq is None else dq
    dk = torch.empty(k.shape, dtype=torch.float32, device=dev) if dk is None else dk
    dv = torch.empty(v.shape, dtype=torch.float32, device=dev) if dv is None else dv
    _check_tensor("dq", dq, torch.float32, q.shape, dev)
    _check_tensor("dk", dk, torch.float32, k.shape, dev)
    _check_tensor("dv", dv, torch.float32, k.shape, dev)
    wsb = attn_bwd_workspace_bytes(B, K, G, T, S, H)
    if workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    _check_workspace(workspace, dev)
    if head_mask is not None:
        if window is not None or prefix != 0:
            raise ValueError("head_mask excludes window and prefix")
        _check_head_mask(head_mask, K, G, dev)
        rc = load_library().attn_bwd_head_masks(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq),
                                                _ptr(dk), _ptr(dv), _ptr(q_seg), _ptr(kv_seg), B, K, G, T, S, H, cm,
                                                _ptr(head_mask), _ptr(workspace), workspace.numel(),
                                                _stream_handle(dev))
        if rc != GQA_ATTN_OK:
            raise GqaAttnError(rc, "attn_bwd_head_masks")
        return dq, dk, dv
    if window is not None or prefix != 0:
        wl, wr = (-1, -1) if window is None else (int(window[0]), int(window[1]))
        rc = load_library().attn_bwd_mask(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq),
                                          _ptr(dk), _ptr(dv), _ptr(q_seg), _ptr(kv_seg), B, K, G, T, S, H, cm,
                                          wl, wr, int(prefix), _ptr(workspace), workspace.numel(),
                                          _stream_handle(dev))
        if rc != GQA_ATTN_OK:
            raise GqaAttnError(rc, "attn_bwd_mask")
        return dq, dk, dv
    rc = load_library().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
                                 _ptr(dv), _ptr(q_seg), _ptr(kv_seg), B, K, G, T, S, H, cm,
                                 _ptr(workspace), workspace.numel(), _stream_handle(dev))
    if rc != GQA_ATTN_OK:
        raise GqaAttnError(rc, "attn_bwd")
    return dq, dk, dv
