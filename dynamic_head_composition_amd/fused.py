"""The attention block's main attention with the Lightweight DC layer fused in
(forward): thin Python binding over the C ABI of libldc.so
(include/ldc_fused.h).

Argument marshalling only (device pointers of torch tensors, the current HIP
stream, the workspace); every step runs in the HIP kernels, and the calls
raise when the library is missing.

    o = fwd(q, k, v, c, g, doc_ids)     # main attention + Lightweight DC, [T,H,d] float32
    o, saved = fwd(q, k, v, c, g, doc_ids, save=True)   # also the layer's saved state for ldc.bwd
    m = main_fwd(q, k, v, doc_ids)      # the main attention alone

The main attention is causal attention of each head over the query's own run
of equal document ids; the reading of the AITNT page "一个国产AI小透明，连续两次
刷新NanoGPT Speedrun世界纪录" (section "第二刀-砍层内", Lightweight DC paragraph)
is in include/ldc_fused.h.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

from . import DEFAULT_WINDOW, LDCError, _check, _dtype_code, _torch, load_library

__all__ = ["fwd", "main_fwd", "workspace_bytes", "main_workspace_bytes"]


def workspace_bytes(dtype_code: int, T: int, H: int, d: int, window: int = DEFAULT_WINDOW) -> int:
    """Bytes of ldc_fused_fwd's workspace (its first ldc.saved_bytes(...) bytes
    receive the layer's saved state)."""
    return int(load_library().ldc_fused_fwd_workspace_bytes(dtype_code, T, H, d, window))


def main_workspace_bytes(T: int) -> int:
    return int(load_library().ldc_main_attention_workspace_bytes(T))


def _out(q, out):
    torch = _torch()
    o = torch.empty(q.shape, dtype=torch.float32, device=q.device) if out is None else out
    if o.shape != q.shape or o.dtype != torch.float32 or not o.is_contiguous() or o.device != q.device:
        raise ValueError("out must be a contiguous float32 tensor shaped like q, on q's device")
    return o


def _ws(q, need, workspace):
    torch = _torch()
    if workspace is None:
        return torch.empty(max(16, need), dtype=torch.uint8, device=q.device)
    if workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    return workspace


def _check_main(q, k, v, doc):
    torch = _torch()
    if q.dim() != 3:
        raise ValueError("q must be [T, H, d]")
    T, H, d = q.shape
    for name, x in (("k", k), ("v", v)):
        if x.shape != q.shape or x.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    if doc.shape != (T,) or doc.dtype != torch.int32:
        raise ValueError("doc_ids must be int32 [T]")
    for name, x in (("q", q), ("k", k), ("v", v), ("doc_ids", doc)):
        if not x.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if x.device != q.device:
            raise ValueError(f"{name} is on another device")
    return T, H, d


def fwd(q, k, v, c, g, doc_ids, window: int = DEFAULT_WINDOW, scale: Optional[float] = None, out=None,
        workspace=None, save: bool = False, stream=None):
    """O[T,H,d] float32: the block's main attention plus the Lightweight DC
    layer.  With save=True, (O, saved): the workspace's leading bytes, the
    layer's saved state as ldc.fwd writes it (pass it to ldc.bwd)."""
    torch = _torch()
    lib = load_library()
    T, H, d = _check(q, k, v, c, g, doc_ids)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = _dtype_code(q)
    need = int(lib.ldc_fused_fwd_workspace_bytes(code, T, H, d, window))
    st_obj = torch.cuda.current_stream(q.device) if stream is None else stream
    with torch.cuda.stream(st_obj):
        o = _out(q, out)
        ws = _ws(q, need, workspace)
    st = lib.ldc_fused_fwd(code, T, H, d, window, float(scale), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                           c.data_ptr(), g.data_ptr(), doc_ids.data_ptr(), o.data_ptr(), ws.data_ptr(), need,
                           ctypes.c_void_p(st_obj.cuda_stream))
    if st != 0:
        raise LDCError(st, "ldc_fused_fwd")
    if save:
        from . import saved_bytes
        return o, ws.view(torch.uint8).reshape(-1)[:max(16, saved_bytes(code, T, H, d, window))]
    return o


def main_fwd(q, k, v, doc_ids, scale: Optional[float] = None, out=None, workspace=None, stream=None):
    """M[T,H,d] float32: causal attention of each head over the query's own document."""
    torch = _torch()
    lib = load_library()
    T, H, d = _check_main(q, k, v, doc_ids)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = int(lib.ldc_main_attention_workspace_bytes(T))
    st_obj = torch.cuda.current_stream(q.device) if stream is None else stream
    with torch.cuda.stream(st_obj):
        o = _out(q, out)
        ws = _ws(q, need, workspace)
    st = lib.ldc_main_attention_fwd(_dtype_code(q), T, H, d, float(scale), q.data_ptr(), k.data_ptr(),
                                    v.data_ptr(), doc_ids.data_ptr(), o.data_ptr(), ws.data_ptr(), need,
                                    ctypes.c_void_p(st_obj.cuda_stream))
    if st != 0:
        raise LDCError(st, "ldc_main_attention_fwd")
    return o
