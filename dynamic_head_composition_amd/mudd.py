"""MUDD layer mixing through the C ABI of libldc.so (include/mudd.h).

Argument marshalling only: every element of the mix is computed by the HIP
kernels; if the library is missing the calls raise.

    ys = fwd(xs, a)              # W float32 tensors [T, dm]
    dxs, da = bwd(xs, a, dys)    # J float32 tensors [T, dm], float32 [T, W, J]
    ys = mudd_mix(xs, a)         # autograd-aware: W tensors in the dtype of xs

xs: J tensors [T, dm] (bfloat16 or float32, one dtype), a: float32 [T, W, J],
dys: W tensors [T, dm] in the dtype of xs.  The mix is the one the AITNT page
"一个国产AI小透明，连续两次刷新NanoGPT Speedrun世界纪录" describes in section
"第一刀—砍层间": Y_w[t] = sum_j A[t, w, j] X_j[t].
"""
from __future__ import annotations

import ctypes

from . import LDC_BF16, LDC_F32, LDCError, load_library

__all__ = ["fwd", "bwd", "mudd_mix", "MuddFunction", "MAX_STREAMS", "MAX_WAYS", "MAX_DIM"]

MAX_STREAMS, MAX_WAYS, MAX_DIM = 16, 4, 16384


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return LDC_BF16
    if t.dtype == torch.float32:
        return LDC_F32
    raise TypeError(f"streams must be bfloat16 or float32, got {t.dtype}")


def _ptrs(ts):
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = t.data_ptr()
    return arr


def _check(xs, a, dys=None):
    import torch
    if len(xs) == 0:
        raise ValueError("at least one stream")
    T, dm = xs[0].shape
    for x in xs:
        if x.shape != (T, dm) or x.dtype != xs[0].dtype:
            raise ValueError("streams must share shape [T, dm] and dtype")
    if a.dtype != torch.float32 or a.dim() != 3 or a.shape[0] != T or a.shape[2] != len(xs):
        raise ValueError("a must be float32 [T, W, J]")
    for d in dys or ():
        if d.shape != (T, dm) or d.dtype != xs[0].dtype:
            raise ValueError("dys must match the streams in shape and dtype")
    if dys is not None and len(dys) != a.shape[1]:
        raise ValueError("one upstream gradient per way")
    for t in list(xs) + [a] + list(dys or ()):
        if not t.is_cuda or not t.is_contiguous() or t.device != xs[0].device:
            raise ValueError("inputs must be contiguous tensors on one device")
    return T, dm, a.shape[1], len(xs)


def _stream(dev, stream):
    """The stream to run on (torch's current one by default)."""
    import torch
    return torch.cuda.current_stream(dev) if stream is None else stream


def fwd(xs, a, out=None, stream=None):
    """The W mixes Y_w = sum_j A[:, w, j] X_j, float32 [T, dm] each."""
    import torch
    lib = load_library()
    T, dm, W, J = _check(xs, a)
    s = _stream(a.device, stream)
    with torch.cuda.stream(s):  # allocated on the stream that uses them
        ys = out if out is not None else [torch.empty((T, dm), dtype=torch.float32, device=a.device)
                                          for _ in range(W)]
    st = lib.mudd_fwd(_dtype_code(xs[0]), T, dm, W, J, _ptrs(xs), a.data_ptr(), _ptrs(ys),
                      ctypes.c_void_p(s.cuda_stream))
    if st != 0:
        raise LDCError(st, "mudd_fwd")
    return ys


def bwd(xs, a, dys, out=None, stream=None):
    """(dX_j for every stream, float32 [T, dm]; dA float32 [T, W, J])."""
    import torch
    lib = load_library()
    T, dm, W, J = _check(xs, a, dys)
    s = _stream(a.device, stream)
    with torch.cuda.stream(s):
        if out is None:
            out = ([torch.empty((T, dm), dtype=torch.float32, device=a.device) for _ in range(J)],
                   torch.empty((T, W, J), dtype=torch.float32, device=a.device))
    dxs, da = out
    st = lib.mudd_bwd(_dtype_code(xs[0]), T, dm, W, J, _ptrs(xs), a.data_ptr(), _ptrs(dys),
                      _ptrs(dxs), da.data_ptr(), ctypes.c_void_p(s.cuda_stream))
    if st != 0:
        raise LDCError(st, "mudd_bwd")
    return dxs, da


def _make_function():
    import torch

    class MuddFunction(torch.autograd.Function):
        """Autograd wrapper: forward = mudd_fwd, backward = mudd_bwd.  The
        mixes stay float32 (rounding them to bf16 would add the storage error
        to every output); stream gradients take the dtype of the streams."""

        @staticmethod
        def forward(ctx, a, *xs):
            ys = fwd(list(xs), a)
            ctx.save_for_backward(a, *xs)
            return tuple(ys)

        @staticmethod
        def backward(ctx, *dys):
            a, *xs = ctx.saved_tensors
            dys = [(torch.zeros_like(xs[0]) if d is None else d.contiguous().to(xs[0].dtype)) for d in dys]
            dxs, da = bwd(xs, a, dys)
            return (da,) + tuple(d.to(xs[0].dtype) for d in dxs)

    return MuddFunction


_fn = None


def __getattr__(name):
    global _fn
    if name == "MuddFunction":
        if _fn is None:
            _fn = _make_function()
        return _fn
    raise AttributeError(name)


def mudd_mix(xs, a):
    """The W mixes of the streams `xs` with weights `a` [T, W, J], through
    autograd (gradients flow to every stream and to the weights)."""
    return list(__getattr__("MuddFunction").apply(a, *xs))
