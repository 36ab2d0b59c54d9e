"""Full DCMHA composition on the Lightweight DC window: thin Python binding
over the C ABI of libldc.so (include/dcmha.h).

Argument marshalling only (device pointers of torch tensors, the current HIP
stream); every step runs in the HIP kernels, and the calls raise when the
library is missing.

    o = fwd(q, k, v, cs, cw, doc_ids)                       # [T,H,d] float32
    o, saved = fwd(q, k, v, cs, cw, doc_ids, save=True)
    dq, dk, dv, dcs, dcw = bwd(q, k, v, cs, cw, doc_ids, saved, do)
    o = dcmha_attention(q, k, v, cs, cw, doc_ids)            # autograd-aware

cs, cw: [T, H, H] float32 score and weight compositions of each query (row =
target head, column = source head), as the AITNT page "一个国产AI小透明，连续两次
刷新NanoGPT Speedrun世界纪录" (section "第二刀-砍层内", DCMHA paragraph)
describes the Compose module; the full definition is in include/dcmha.h.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

from . import DEFAULT_WINDOW, LDCError, _buf, _dtype_code, _torch, load_library

__all__ = ["fwd", "bwd", "dcmha_attention", "saved_bytes", "workspace_bytes", "MAX_HEADS"]

MAX_HEADS = 6


def saved_bytes(dtype: int, T: int, H: int, d: int, window: int = DEFAULT_WINDOW) -> int:
    return int(load_library().dcmha_saved_bytes(dtype, T, H, d, window))


def workspace_bytes(dtype: int, T: int, H: int, d: int, window: int = DEFAULT_WINDOW) -> int:
    return int(load_library().dcmha_bwd_workspace_bytes(dtype, T, H, d, window))


def _check(q, k, v, cs, cw, doc, do=None):
    torch = _torch()
    if q.dim() != 3:
        raise ValueError("q must be [T, H, d]")
    T, H, d = q.shape
    for name, x in (("k", k), ("v", v)) + ((("do", do),) if do is not None else ()):
        if x.shape != q.shape or x.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    for name, x in (("cs", cs), ("cw", cw)):
        if tuple(x.shape) != (T, H, H) or x.dtype != torch.float32:
            raise ValueError(f"{name} must be float32 [T, H, H]")
    if doc.shape != (T,) or doc.dtype != torch.int32:
        raise ValueError("doc_ids must be int32 [T]")
    for name, x in (("q", q), ("k", k), ("v", v), ("cs", cs), ("cw", cw), ("doc_ids", doc)) + \
            ((("do", do),) if do is not None else ()):
        if not x.is_cuda or not x.is_contiguous() or x.device != q.device:
            raise ValueError(f"{name} must be a contiguous device tensor on q's device")
    return T, H, d


def fwd(q, k, v, cs, cw, doc_ids, window: int = DEFAULT_WINDOW, scale: Optional[float] = None,
        out=None, save: bool = False, saved=None, stream=None):
    """O[T,H,d] float32; with save=True (or a `saved` buffer) also the state
    bwd needs, returned as (O, saved).  Enqueued on `stream` (default: the
    current stream); tensors this call allocates are allocated on it."""
    torch = _torch()
    lib = load_library()
    T, H, d = _check(q, k, v, cs, cw, doc_ids)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st_obj = torch.cuda.current_stream(q.device) if stream is None else stream
    with torch.cuda.stream(st_obj):
        o = torch.empty(q.shape, dtype=torch.float32, device=q.device) if out is None else out
        if save and saved is None:
            saved = torch.empty(max(16, saved_bytes(_dtype_code(q), T, H, d, window)), dtype=torch.uint8,
                                device=q.device)
    if o.shape != q.shape or o.dtype != torch.float32 or not o.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor shaped like q")
    sp, sn = _buf(saved)
    st = lib.dcmha_fwd(_dtype_code(q), T, H, d, window, float(scale), q.data_ptr(), k.data_ptr(),
                       v.data_ptr(), cs.data_ptr(), cw.data_ptr(), doc_ids.data_ptr(), o.data_ptr(),
                       sp, sn, ctypes.c_void_p(st_obj.cuda_stream))
    if st != 0:
        raise LDCError(st, "dcmha_fwd")
    return (o, saved) if saved is not None else o


def bwd(q, k, v, cs, cw, doc_ids, saved, do, window: int = DEFAULT_WINDOW,
        scale: Optional[float] = None, out=None, workspace=None, stream=None, part: str = "all"):
    """(dQ, dK, dV, dCS, dCW), float32.  `saved` from fwd(..., save=True) on the
    same inputs, or None (the state is then recomputed into the workspace).
    part="q"/"kv" runs one of the two kernels (part="kv" needs the workspace a
    part="q" call filled)."""
    torch = _torch()
    lib = load_library()
    T, H, d = _check(q, k, v, cs, cw, doc_ids, do)
    if part not in ("all", "q", "kv"):
        raise ValueError("part must be 'all', 'q' or 'kv'")
    if part == "kv" and workspace is None:
        raise ValueError("part='kv' reads the dS bands a part='q' call wrote: pass that workspace")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st_obj = torch.cuda.current_stream(q.device) if stream is None else stream
    with torch.cuda.stream(st_obj):
        if out is None:
            f32 = dict(dtype=torch.float32, device=q.device)
            out = (torch.empty((T, H, d), **f32), torch.empty((T, H, d), **f32),
                   torch.empty((T, H, d), **f32), torch.empty((T, H, H), **f32),
                   torch.empty((T, H, H), **f32))
        if workspace is None:
            workspace = torch.empty(max(16, workspace_bytes(_dtype_code(q), T, H, d, window)),
                                    dtype=torch.uint8, device=q.device)
    for name, x, shape in zip(("dq", "dk", "dv", "dcs", "dcw"), out, ((T, H, d),) * 3 + ((T, H, H),) * 2):
        if tuple(x.shape) != shape or x.dtype != torch.float32 or not x.is_contiguous() or x.device != q.device:
            raise ValueError(f"{name} must be a contiguous float32 {list(shape)} tensor on {q.device}")
    dq, dk, dv, dcs, dcw = out
    sp, sn = _buf(saved)
    wp, wn = _buf(workspace)
    name = {"all": "dcmha_bwd", "q": "dcmha_bwd_q", "kv": "dcmha_bwd_kv"}[part]
    st = getattr(lib, name)(_dtype_code(q), T, H, d, window, float(scale), q.data_ptr(), k.data_ptr(),
                            v.data_ptr(), cs.data_ptr(), cw.data_ptr(), doc_ids.data_ptr(), sp, sn,
                            do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dcs.data_ptr(),
                            dcw.data_ptr(), wp, wn, ctypes.c_void_p(st_obj.cuda_stream))
    if st != 0:
        raise LDCError(st, name)
    return dq, dk, dv, dcs, dcw


def _make_function():
    torch = _torch()

    class DCMHAFunction(torch.autograd.Function):
        """Autograd wrapper: O (float32) from dcmha_fwd, gradients from dcmha_bwd."""

        @staticmethod
        def forward(ctx, q, k, v, cs, cw, doc_ids, window=DEFAULT_WINDOW, scale=None):
            o, saved = fwd(q, k, v, cs, cw, doc_ids, window=window, scale=scale, save=True)
            ctx.save_for_backward(q, k, v, cs, cw, doc_ids, saved)
            ctx.window, ctx.scale = window, scale
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, cs, cw, doc_ids, saved = ctx.saved_tensors
            dq, dk, dv, dcs, dcw = bwd(q, k, v, cs, cw, doc_ids, saved, do.to(q.dtype).contiguous(),
                                       window=ctx.window, scale=ctx.scale)
            return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), dcs, dcw, None, None, None

    return DCMHAFunction


_FN = None


def dcmha_attention(q, k, v, cs, cw, doc_ids, window: int = DEFAULT_WINDOW, scale: Optional[float] = None):
    """Autograd-aware DCMHA layer: O float32 [T,H,d]."""
    global _FN
    if _FN is None:
        _FN = _make_function()
    return _FN.apply(q, k, v, cs, cw, doc_ids, window, scale)
