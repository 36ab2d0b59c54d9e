"""Lightweight DC (dynamically composable multi-head) attention on MI355X.

Thin Python binding over the C ABI of libldc.so (include/ldc.h).  This module
only marshals arguments: shapes, dtypes and device pointers of torch tensors,
and the current HIP stream.  Every step of the layer runs in the HIP kernels;
there is no fallback — if the library is missing the calls raise.

    o = fwd(q, k, v, c, g, doc_ids)                        # [T,H,d] float32
    o, saved = fwd(q, k, v, c, g, doc_ids, save=True)      # + state for bwd
    dq, dk, dv, dc, dg = bwd(q, k, v, c, g, doc_ids, saved, do)
    o = ldc_attention(q, k, v, c, g, doc_ids)              # autograd-aware

The layer is the one the AITNT page "一个国产AI小透明，连续两次刷新NanoGPT
Speedrun世界纪录" describes in section "第二刀-砍层内" (Lightweight DC
paragraph); the exact definition, with the readings taken where the page is
silent, is in include/ldc.h.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

__all__ = ["fwd", "bwd", "bwd_noalloc", "noalloc_max_workspace", "ldc_attention", "LDCFunction", "LDCError", "load_library",
           "workspace_bytes", "saved_bytes", "status_str", "version", "LIB_PATH",
           "LDC_BF16", "LDC_F32"]

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libldc.so")
LDC_BF16, LDC_F32 = 0, 1
DEFAULT_WINDOW = 112

_lib = None


class LDCError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libldc.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m dynamic_head_composition_amd.build`")
    # torch first: its HIP runtime is then the one libldc.so binds to, so the
    # streams and device memory torch hands over belong to the runtime that
    # launches the kernels (loading the library first, then torch, left the
    # launches failing with LDC_ERR_HIP in one process)
    import torch  # noqa: F401
    lib = ctypes.CDLL(p)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.ldc_fwd.argtypes = [i32, i64, i32, i32, i32, f32] + [vp] * 7 + [vp, sz, vp]
    lib.ldc_fwd.restype = i32
    for nm in ("ldc_bwd", "ldc_bwd_q", "ldc_bwd_kv"):
        getattr(lib, nm).argtypes = ([i32, i64, i32, i32, i32, f32] + [vp] * 6 + [vp, sz]
                                     + [vp] * 6 + [vp, sz, vp])
        getattr(lib, nm).restype = i32
    lib.ldc_bwd_noalloc.argtypes = ([i32, i64, i32, i32, i32, f32] + [vp] * 6 + [vp, sz]
                                    + [vp] * 6 + [vp])
    lib.ldc_bwd_noalloc.restype = i32
    lib.ldc_bwd_noalloc_max_workspace.argtypes = []
    lib.ldc_bwd_noalloc_max_workspace.restype = sz
    for nm in ("ldc_bwd_workspace_bytes", "ldc_saved_bytes"):
        getattr(lib, nm).argtypes = [i32, i64, i32, i32, i32]
        getattr(lib, nm).restype = sz
    lib.ldc_status_str.argtypes = [i32]
    lib.ldc_status_str.restype = ctypes.c_char_p
    lib.ldc_version.argtypes = []
    lib.ldc_version.restype = i32
    lib.dcmha_fwd.argtypes = [i32, i64, i32, i32, i32, f32] + [vp] * 7 + [vp, sz, vp]
    lib.dcmha_fwd.restype = i32
    for nm in ("dcmha_bwd", "dcmha_bwd_q", "dcmha_bwd_kv"):
        getattr(lib, nm).argtypes = ([i32, i64, i32, i32, i32, f32] + [vp] * 6 + [vp, sz]
                                     + [vp] * 6 + [vp, sz, vp])
        getattr(lib, nm).restype = i32
    for nm in ("dcmha_saved_bytes", "dcmha_bwd_workspace_bytes"):
        getattr(lib, nm).argtypes = [i32, i64, i32, i32, i32]
        getattr(lib, nm).restype = sz
    lib.ldc_cg_fwd.argtypes = [i32, i64, i32, i32] + [vp] * 5 + [vp]
    lib.ldc_fused_fwd.argtypes = [i32, i64, i32, i32, i32, f32] + [vp] * 7 + [vp, sz, vp]
    lib.ldc_fused_fwd.restype = i32
    lib.ldc_fused_fwd_workspace_bytes.argtypes = [i32, i64, i32, i32, i32]
    lib.ldc_fused_fwd_workspace_bytes.restype = sz
    lib.ldc_main_attention_fwd.argtypes = [i32, i64, i32, i32, f32] + [vp] * 5 + [vp, sz, vp]
    lib.ldc_main_attention_fwd.restype = i32
    lib.ldc_main_attention_workspace_bytes.argtypes = [i64]
    lib.ldc_main_attention_workspace_bytes.restype = sz
    lib.ldc_cg_fwd.restype = i32
    lib.ldc_cg_bwd.argtypes = [i32, i64, i32, i32] + [vp] * 8 + [vp, sz, vp]
    lib.ldc_cg_bwd.restype = i32
    lib.ldc_cg_bwd_workspace_bytes.argtypes = [i32, i64, i32, i32]
    lib.ldc_cg_bwd_workspace_bytes.restype = sz
    lib.mudd_fwd.argtypes = [i32, i64, i32, i32, i32, vp, vp, vp, vp]
    lib.mudd_fwd.restype = i32
    lib.mudd_bwd.argtypes = [i32, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    lib.mudd_bwd.restype = i32
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().ldc_status_str(int(status)).decode()


def version() -> int:
    return int(load_library().ldc_version())


def workspace_bytes(dtype: int, T: int, H: int, d: int, window: int = DEFAULT_WINDOW) -> int:
    return int(load_library().ldc_bwd_workspace_bytes(dtype, T, H, d, window))


def saved_bytes(dtype: int, T: int, H: int, d: int, window: int = DEFAULT_WINDOW) -> int:
    return int(load_library().ldc_saved_bytes(dtype, T, H, d, window))


# ---------------------------------------------------------------------------
# torch-tensor front end (PyTorch provides device memory and the stream only)
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return LDC_BF16
    if t.dtype == torch.float32:
        return LDC_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _check(q, k, v, c, g, doc, do=None):
    torch = _torch()
    if q.dim() != 3:
        raise ValueError("q must be [T, H, d]")
    T, H, d = q.shape
    for name, x in (("k", k), ("v", v)) + ((("do", do),) if do is not None else ()):
        if x.shape != q.shape or x.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    for name, x in (("c", c), ("g", g)):
        if x.shape != (T, H) or x.dtype != torch.float32:
            raise ValueError(f"{name} must be float32 [T, H]")
    if doc.shape != (T,) or doc.dtype != torch.int32:
        raise ValueError("doc_ids must be int32 [T]")
    for name, x in (("q", q), ("k", k), ("v", v), ("c", c), ("g", g), ("doc_ids", doc)) + \
            ((("do", do),) if do is not None else ()):
        if not x.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if x.device != q.device:
            raise ValueError(f"{name} is on another device")
    return T, H, d


def _buf(t):
    return (0, 0) if t is None else (t.data_ptr(), t.numel() * t.element_size())


def fwd(q, k, v, c, g, doc_ids, window: int = DEFAULT_WINDOW, scale: Optional[float] = None,
        out=None, save: bool = False, saved=None, stream=None):
    """O[t,h,:] of the layer, float32 [T,H,d].  With save=True (or a `saved`
    buffer) also the state ldc_bwd needs, returned as (O, saved).  Enqueued on
    `stream` (default: torch's current stream), not synchronised; tensors this
    call allocates are allocated on that stream."""
    torch = _torch()
    lib = load_library()
    T, H, d = _check(q, k, v, c, g, doc_ids)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st_obj = torch.cuda.current_stream(q.device) if stream is None else stream
    with torch.cuda.stream(st_obj):
        o = torch.empty(q.shape, dtype=torch.float32, device=q.device) if out is None else out
        if save and saved is None:
            saved = torch.empty(max(16, saved_bytes(_dtype_code(q), T, H, d, window)),
                                dtype=torch.uint8, device=q.device)
    if o.shape != q.shape or o.dtype != torch.float32 or not o.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor shaped like q")
    sp, sn = _buf(saved)
    st = lib.ldc_fwd(_dtype_code(q), T, H, d, window, float(scale),
                     q.data_ptr(), k.data_ptr(), v.data_ptr(), c.data_ptr(), g.data_ptr(),
                     doc_ids.data_ptr(), o.data_ptr(), sp, sn, ctypes.c_void_p(st_obj.cuda_stream))
    if st != 0:
        raise LDCError(st, "ldc_fwd")
    return (o, saved) if saved is not None else o


def bwd(q, k, v, c, g, doc_ids, saved, do, window: int = DEFAULT_WINDOW,
        scale: Optional[float] = None, out=None, workspace=None, stream=None, part: str = "all"):
    """(dQ, dK, dV, dC, dG), all float32, given `saved` from fwd(..., save=True)
    on the same inputs.  part="q" or "kv" runs one of the two backward kernels
    only (ldc_bwd_q / ldc_bwd_kv); "all" runs both.  part="kv" needs the
    `workspace` a part="q" call filled for the same inputs (it reads dPbar
    from there).  Tensors this call allocates are allocated on `stream`, so the
    caching allocator does not hand them out while the kernels still use them."""
    torch = _torch()
    lib = load_library()
    T, H, d = _check(q, k, v, c, g, doc_ids, do)
    if part not in ("all", "q", "kv"):
        raise ValueError("part must be 'all', 'q' or 'kv'")
    if part == "kv" and workspace is None:
        raise ValueError("part='kv' reads the dPbar band a part='q' call wrote: pass that workspace")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st_obj = torch.cuda.current_stream(q.device) if stream is None else stream
    with torch.cuda.stream(st_obj):
        if out is None:
            f32 = dict(dtype=torch.float32, device=q.device)
            out = (torch.empty((T, H, d), **f32), torch.empty((T, H, d), **f32),
                   torch.empty((T, H, d), **f32), torch.empty((T, H), **f32),
                   torch.empty((T, H), **f32))
        if workspace is None:
            need = workspace_bytes(_dtype_code(q), T, H, d, window)
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_grads(out, T, H, d, q.device)
    dq, dk, dv, dc, dg = out
    sp, sn = _buf(saved)
    wp, wn = _buf(workspace)
    entry = {"all": lib.ldc_bwd, "q": lib.ldc_bwd_q, "kv": lib.ldc_bwd_kv}[part]
    st = entry(_dtype_code(q), T, H, d, window, float(scale),
               q.data_ptr(), k.data_ptr(), v.data_ptr(), c.data_ptr(), g.data_ptr(),
               doc_ids.data_ptr(), sp, sn, do.data_ptr(),
               dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dc.data_ptr(), dg.data_ptr(),
               wp, wn, ctypes.c_void_p(st_obj.cuda_stream))
    if st != 0:
        raise LDCError(st, {"all": "ldc_bwd", "q": "ldc_bwd_q", "kv": "ldc_bwd_kv"}[part])
    return dq, dk, dv, dc, dg


def _check_grads(out, T, H, d, device):
    torch = _torch()
    if out is None or len(out) != 5:
        raise ValueError("out must be the five gradient tensors (dq, dk, dv, dc, dg)")
    for name, x, shape in zip(("dq", "dk", "dv", "dc", "dg"), out,
                              ((T, H, d),) * 3 + ((T, H),) * 2):
        if (tuple(x.shape) != shape or x.dtype != torch.float32 or not x.is_contiguous()
                or x.device != device):
            raise ValueError(f"{name} must be a contiguous float32 {list(shape)} tensor on {device}")


def bwd_noalloc(q, k, v, c, g, doc_ids, saved, do, out, window: int = DEFAULT_WINDOW,
                scale: Optional[float] = None, stream=None):
    """ldc_bwd without a caller workspace and without any allocation: the
    library's static per-GPU scratch serves as workspace (ldc_bwd_noalloc).
    `out` = (dq, dk, dv, dc, dg) must be given.  Calls that overlap on one GPU
    race on the scratch: keep them on one stream."""
    torch = _torch()
    lib = load_library()
    T, H, d = _check(q, k, v, c, g, doc_ids, do)
    _check_grads(out, T, H, d, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st_obj = torch.cuda.current_stream(q.device) if stream is None else stream
    dq, dk, dv, dc, dg = out
    sp, sn = _buf(saved)
    st = lib.ldc_bwd_noalloc(_dtype_code(q), T, H, d, window, float(scale),
                             q.data_ptr(), k.data_ptr(), v.data_ptr(), c.data_ptr(), g.data_ptr(),
                             doc_ids.data_ptr(), sp, sn, do.data_ptr(),
                             dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dc.data_ptr(),
                             dg.data_ptr(), ctypes.c_void_p(st_obj.cuda_stream))
    if st != 0:
        raise LDCError(st, "ldc_bwd_noalloc")
    return out


def noalloc_max_workspace() -> int:
    return int(load_library().ldc_bwd_noalloc_max_workspace())


def _make_function():
    torch = _torch()

    class LDCFunction(torch.autograd.Function):
        """Autograd wrapper: forward = ldc_fwd, backward = ldc_bwd.

        O is returned in float32 whatever the input dtype: a bf16 store alone
        would round outputs of magnitude above ~5 by more than the bf16
        tolerance (2e-2).  The incoming gradient is cast to the input dtype
        for the kernels; the gradients of bf16 inputs are then rounded to bf16
        by autograd, which gives a leaf the gradient dtype of the leaf."""

        @staticmethod
        def forward(ctx, q, k, v, c, g, doc_ids, window=DEFAULT_WINDOW, scale=None):
            o, saved = fwd(q, k, v, c, g, doc_ids, window, scale, save=True)
            ctx.save_for_backward(q, k, v, c, g, doc_ids, saved)
            ctx.window, ctx.scale = window, scale
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, c, g, doc, saved = ctx.saved_tensors
            dq, dk, dv, dc, dg = bwd(q, k, v, c, g, doc, saved, do.contiguous().to(q.dtype),
                                     ctx.window, ctx.scale)
            return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), dc, dg, None, None, None

    return LDCFunction


_fn = None


def __getattr__(name):
    global _fn
    if name == "LDCFunction":
        if _fn is None:
            _fn = _make_function()
        return _fn
    raise AttributeError(name)


def ldc_attention(q, k, v, c, g, doc_ids, window: int = DEFAULT_WINDOW, scale: Optional[float] = None):
    return __getattr__("LDCFunction").apply(q, k, v, c, g, doc_ids, window, scale)
