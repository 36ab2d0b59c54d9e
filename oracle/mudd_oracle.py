"""Plain fp64 CPU oracle of multiway dynamic dense (MUDD) layer mixing.

TEST INFRASTRUCTURE.  Only tests, the smoke check and the CPU-baseline leg of
the benchmark may import this module.  It shares no code with the HIP path and
imports nothing from it.

What is computed (AITNT page "一个国产AI小透明，连续两次刷新NanoGPT Speedrun
世界纪录", section "第一刀—砍层间", and the MUDD remarks in section "和业界其他
工作的联系"): instead of one fixed residual path, the input a layer receives is
a per-token mix of the outputs of earlier layers, with weights generated from
the current hidden state; the weights are not normalised by a softmax and may
be negative, so a layer can amplify, suppress or cancel an earlier one.  The
full method keeps four such mixes ("ways": the Q, K, V and residual inputs);
the skip-connection variant keeps one.  Readings taken where the page is
silent:

* the mixed streams X_0 .. X_{J-1} are [T, dm] tensors (token-major), one per
  earlier layer, the embedding included;
* the weights A[t, w, j] (token t, way w, stream j) are inputs: their
  generator sits upstream of the mix, as the page does not give its form;
* each way is the plain weighted sum, with no bias, normalisation or
  activation.

Forward, per token t and way w:
    Y_w[t, :] = sum_j A[t, w, j] X_j[t, :]

Backward (the mix is bilinear in A and the X_j), given dY_w:
    dX_j[t, :]   = sum_w A[t, w, j] dY_w[t, :]
    dA[t, w, j]  = <dY_w[t, :], X_j[t, :]>

Inputs are upcast to float64 first; the sums are numpy float64 operations.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _check(xs: Sequence[np.ndarray], a: np.ndarray) -> Tuple[int, int, int, int]:
    if len(xs) == 0:
        raise ValueError("at least one stream")
    T, dm = xs[0].shape
    for x in xs:
        if x.shape != (T, dm):
            raise ValueError("every stream must be [T, dm]")
    if a.ndim != 3 or a.shape[0] != T or a.shape[2] != len(xs):
        raise ValueError("weights must be [T, W, J]")
    return T, dm, a.shape[1], len(xs)


def forward(xs: Sequence[np.ndarray], a: np.ndarray) -> np.ndarray:
    """Y [W, T, dm]: Y[w, t] = sum_j a[t, w, j] * xs[j][t]."""
    xs = [_f64(x) for x in xs]
    a = _f64(a)
    T, dm, W, J = _check(xs, a)
    y = np.zeros((W, T, dm))
    for w in range(W):
        for j in range(J):
            y[w] += a[:, w, j][:, None] * xs[j]
    return y


def backward(xs: Sequence[np.ndarray], a: np.ndarray,
             dys: Sequence[np.ndarray]) -> Tuple[np.ndarray, np.ndarray]:
    """(dX [J, T, dm], dA [T, W, J]) for upstream gradients dys[w] = dL/dY_w."""
    xs = [_f64(x) for x in xs]
    a = _f64(a)
    dys = [_f64(d) for d in dys]
    T, dm, W, J = _check(xs, a)
    if len(dys) != W or any(d.shape != (T, dm) for d in dys):
        raise ValueError("one [T, dm] upstream gradient per way")
    dx = np.zeros((J, T, dm))
    da = np.zeros((T, W, J))
    for j in range(J):
        for w in range(W):
            dx[j] += a[:, w, j][:, None] * dys[w]
            da[:, w, j] = np.sum(dys[w] * xs[j], axis=1)
    return dx, da
