"""Generator of the Lightweight DC weights C and G from the layer's input
hidden state: thin Python binding over include/ldc_cg.h (argument
marshalling only; the kernels do the work and the calls raise when the
library is missing).

    c, g = fwd(x, wc, wg)                       # [T, H] float32 each
    dx, dwc, dwg = bwd(x, wc, wg, dc, dg)        # float32

x [T, dm] and wc, wg [dm, H] in bfloat16 or float32 (the same dtype).  The
reading of the AITNT page (section "第二刀-砍层内": the composition is decided
from the current input) is C = x WC, G = x WG; see include/ldc_cg.h.
"""
from __future__ import annotations

import ctypes

from . import LDCError, _dtype_code, _torch, load_library

__all__ = ["fwd", "bwd", "workspace_bytes"]


def workspace_bytes(dtype: int, T: int, dm: int, H: int) -> int:
    return int(load_library().ldc_cg_bwd_workspace_bytes(dtype, T, dm, H))


def _check(x, wc, wg):
    if x.dim() != 2 or wc.dim() != 2 or wc.shape != wg.shape or wc.shape[0] != x.shape[1]:
        raise ValueError("x must be [T, dm] and wc, wg [dm, H]")
    for name, t in (("x", x), ("wc", wc), ("wg", wg)):
        if t.dtype != x.dtype or not t.is_cuda or not t.is_contiguous() or t.device != x.device:
            raise ValueError(f"{name} must be a contiguous device tensor of x's dtype and device")
    return x.shape[0], x.shape[1], wc.shape[1]


def fwd(x, wc, wg, out=None, stream=None):
    torch = _torch()
    lib = load_library()
    T, dm, H = _check(x, wc, wg)
    st_obj = torch.cuda.current_stream(x.device) if stream is None else stream
    with torch.cuda.stream(st_obj):
        if out is None:
            out = (torch.empty((T, H), dtype=torch.float32, device=x.device),
                   torch.empty((T, H), dtype=torch.float32, device=x.device))
    c, g = out
    for name, t in (("c", c), ("g", g)):
        if tuple(t.shape) != (T, H) or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 [T, H] tensor")
    st = lib.ldc_cg_fwd(_dtype_code(x), T, dm, H, x.data_ptr(), wc.data_ptr(), wg.data_ptr(), c.data_ptr(),
                        g.data_ptr(), ctypes.c_void_p(st_obj.cuda_stream))
    if st != 0:
        raise LDCError(st, "ldc_cg_fwd")
    return c, g


def bwd(x, wc, wg, dc, dg, out=None, workspace=None, stream=None):
    torch = _torch()
    lib = load_library()
    T, dm, H = _check(x, wc, wg)
    for name, t in (("dc", dc), ("dg", dg)):
        if tuple(t.shape) != (T, H) or t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous float32 [T, H] device tensor")
    st_obj = torch.cuda.current_stream(x.device) if stream is None else stream
    f32 = dict(dtype=torch.float32, device=x.device)
    with torch.cuda.stream(st_obj):
        if out is None:
            out = (torch.empty((T, dm), **f32), torch.empty((dm, H), **f32), torch.empty((dm, H), **f32))
        if workspace is None:
            workspace = torch.empty(max(16, workspace_bytes(_dtype_code(x), T, dm, H)), dtype=torch.uint8,
                                    device=x.device)
    dx, dwc, dwg = out
    for name, t, shape in (("dx", dx, (T, dm)), ("dwc", dwc, (dm, H)), ("dwg", dwg, (dm, H))):
        if tuple(t.shape) != shape or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 {list(shape)} tensor")
    st = lib.ldc_cg_bwd(_dtype_code(x), T, dm, H, x.data_ptr(), wc.data_ptr(), wg.data_ptr(), dc.data_ptr(),
                        dg.data_ptr(), dx.data_ptr(), dwc.data_ptr(), dwg.data_ptr(), workspace.data_ptr(),
                        workspace.numel(), ctypes.c_void_p(st_obj.cuda_stream))
    if st != 0:
        raise LDCError(st, "ldc_cg_bwd")
    return dx, dwc, dwg
