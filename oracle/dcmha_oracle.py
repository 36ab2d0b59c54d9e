"""Plain fp64 CPU oracle of the full dynamically composable multi-head
attention (DCMHA) composition, on the same local, document-cut window as the
Lightweight DC layer.

TEST INFRASTRUCTURE.  Only tests, the smoke check and the CPU-baseline leg of
the benchmark may import this module.  It shares no code with the HIP path,
imports nothing from it, and imports nothing from the other oracle modules
(the tests compare it with them as independent implementations).

What is computed (AITNT page "一个国产AI小透明，连续两次刷新NanoGPT
Speedrun世界纪录", section "第二刀-砍层内", DCMHA paragraph): a Compose module
transforms the attention scores and the attention weights across heads, with
a transformation decided by the current input.  Readings taken where the page
is silent:

* both transforms are linear maps over the head axis applied at every
  (query, key) pair: the scores before the softmax with an H x H matrix
  CS[t], the weights after it with an H x H matrix CW[t]; row h of a matrix
  gives the target head h, column h' the source head h';
* the matrices are indexed by the query token t (one pair per query, as the
  Lightweight DC weights are) and are inputs of the layer (whatever produces
  them from the hidden state lies outside it); any real values, no
  renormalisation;
* the window, document cut and softmax scale are the Lightweight DC ones:
  key s is admitted for query t iff t-W+1 <= s <= t and doc[s] == doc[t];
  scale sigma = 1/sqrt(d) unless given.

Forward, per query t (A(t) its admitted keys, never empty: it holds t):
    S_h[t,s]  = sigma <Q[t,h], K[s,h]>                   s in A(t)
    Z_h[t,s]  = sum_h' CS[t,h,h'] S_h'[t,s]              (score composition)
    P_h[t,:]  = softmax over A(t) of Z_h[t,:]
    R_h[t,s]  = sum_h' CW[t,h,h'] P_h'[t,s]              (weight composition)
    O[t,h]    = sum_s R_h[t,s] V[s,h]

Backward (chain rule through the definitions above, given dO):
    dR_h[t,s] = <dO[t,h], V[s,h]>
    dV[s,h]  += R_h[t,s] dO[t,h]
    dCW[t,h,h'] = sum_s dR_h[t,s] P_h'[t,s]
    dP_h'     = sum_h CW[t,h,h'] dR_h
    dZ_h      = P_h (dP_h - sum_s dP_h[t,s] P_h[t,s])    (softmax Jacobian)
    dCS[t,h,h'] = sum_s dZ_h[t,s] S_h'[t,s]
    dS_h'     = sum_h CS[t,h,h'] dZ_h
    dQ[t,h]   = sigma sum_s dS_h[t,s] K[s,h]
    dK[s,h]  += sigma dS_h[t,s] Q[t,h]

The computation walks the queries one at a time, gathers the admitted keys,
and evaluates the formulas with float64 numpy products over the head axis.
All inputs are upcast to float64 first.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def window_keys(doc: np.ndarray, t: int, window: int) -> np.ndarray:
    """Indices of the keys admitted for query t, ascending."""
    s = np.arange(max(0, t - window + 1), t + 1)
    return s[doc[s] == doc[t]]


def _softmax_rows(z: np.ndarray) -> np.ndarray:
    m = z.max(axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / e.sum(axis=-1, keepdims=True)


def _query_maps(q, k, cs, cw, doc, t, window, scale):
    """(keys, S [H,n], P [H,n], R [H,n]) of query t."""
    s = window_keys(doc, t, window)
    S = scale * np.einsum("hd,shd->hs", q[t], k[s])
    P = _softmax_rows(cs[t] @ S)
    R = cw[t] @ P
    return s, S, P, R


def forward(q, k, v, cs, cw, doc, window: int = 112, scale: Optional[float] = None,
            queries=None, return_maps: bool = False):
    """O[T,H,d] (float64).  `queries`: evaluate only these query rows (the
    other rows of O stay 0).  With return_maps, also {t: (keys, S, P, R)}."""
    q, k, v, cs, cw = map(_f64, (q, k, v, cs, cw))
    doc = np.asarray(doc)
    T, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.zeros((T, H, d))
    maps = {}
    for t in (range(T) if queries is None else queries):
        s, S, P, R = _query_maps(q, k, cs, cw, doc, t, window, scale)
        o[t] = np.einsum("hs,shd->hd", R, v[s])
        if return_maps:
            maps[t] = (s, S, P, R)
    return (o, maps) if return_maps else o


def backward(q, k, v, cs, cw, doc, do, window: int = 112, scale: Optional[float] = None):
    """(dQ, dK, dV [T,H,d], dCS, dCW [T,H,H]) in float64."""
    q, k, v, cs, cw, do = map(_f64, (q, k, v, cs, cw, do))
    doc = np.asarray(doc)
    T, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dcs, dcw = np.zeros((T, H, H)), np.zeros((T, H, H))
    for t in range(T):
        s, S, P, R = _query_maps(q, k, cs, cw, doc, t, window, scale)
        dR = np.einsum("hd,shd->hs", do[t], v[s])
        dv[s] += np.einsum("hs,hd->shd", R, do[t])
        dcw[t] = dR @ P.T
        dP = cw[t].T @ dR
        dZ = P * (dP - (dP * P).sum(axis=1, keepdims=True))
        dcs[t] = dZ @ S.T
        dS = cs[t].T @ dZ
        dq[t] = scale * np.einsum("hs,shd->hd", dS, k[s])
        dk[s] += scale * np.einsum("hs,hd->shd", dS, q[t])
    return dq, dk, dv, dcs, dcw
