"""Plain fp64 CPU oracle of the Lightweight DC (LDC) layer.

TEST INFRASTRUCTURE.  Only tests, the smoke check and the CPU-baseline leg of
the benchmark may import this module.  It shares no code with the HIP path and
imports nothing from it.

What the layer computes (AITNT page "一个国产AI小透明，连续两次刷新NanoGPT
Speedrun世界纪录", section "第二刀-砍层内", Lightweight DC paragraph): it reuses
the attention block's Q and K, computes softmax attention per head over a local
window of 112 tokens, then composes the heads' attention maps into one shared
map with dynamic weights, and that shared map acts on each head's Value through
a per-head scale.  Readings taken where the page is silent:

* window membership: key s is in query t's window iff t-W+1 <= s <= t (W keys
  including t itself); keys of another document (doc_ids differ) are masked;
* softmax scale sigma = 1/sqrt(d) unless given;
* the composition is post-softmax only, with weights C[t, h] indexed by the
  query token; C is any real (no renormalisation of the shared map);
* the head scale G[t, h] multiplies head h's output at query t;
* masked entries contribute exactly 0; every window holds t itself, so no row
  is empty.

Forward, per query t (A(t) its admitted keys):
    S_h[t,s] = sigma <Q[t,h], K[s,h]>                         s in A(t)
    P_h[t,:] = softmax over A(t) of S_h[t,:]
    Pbar[t,s] = sum_h C[t,h] P_h[t,s]
    A_h[t]   = sum_s Pbar[t,s] V[s,h]
    O[t,h]   = G[t,h] A_h[t]

Backward (chain rule through the definitions above, given dO):
    dG[t,h]   = <dO[t,h], A_h[t]>
    B_h[t,s]  = <dO[t,h], V[s,h]>
    dPbar     = sum_h G[t,h] B_h[t,s]
    dV[s,h]  += G[t,h] Pbar[t,s] dO[t,h]
    dC[t,h]   = sum_s P_h[t,s] dPbar[t,s]       (dP_h = C[t,h] dPbar)
    dS_h      = C[t,h] P_h (dPbar - dC[t,h])    (softmax Jacobian applied to dP_h)
    dQ[t,h]   = sigma sum_s dS_h[t,s] K[s,h]
    dK[s,h]  += sigma dS_h[t,s] Q[t,h]

The computation walks query blocks of `block` rows; each block gathers its key
band [t0-W+1, t1), builds the admission mask, and evaluates the formulas with
numpy float64 matrix products.  All inputs are upcast to float64 first.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def admitted(doc: np.ndarray, t_idx: np.ndarray, s_idx: np.ndarray, window: int) -> np.ndarray:
    """Boolean [len(t_idx), len(s_idx)]: key s admitted for query t."""
    t = t_idx[:, None]
    s = s_idx[None, :]
    return (s <= t) & (t - s < window) & (doc[s_idx][None, :] == doc[t_idx][:, None])


def _masked_softmax_rows(S: np.ndarray, mask: np.ndarray) -> np.ndarray:
    S = np.where(mask, S, -np.inf)
    m = S.max(axis=-1, keepdims=True)
    e = np.where(mask, np.exp(S - m), 0.0)
    return e / e.sum(axis=-1, keepdims=True)


def _blocks(T: int, window: int, block: int):
    for t0 in range(0, T, block):
        t1 = min(T, t0 + block)
        b0 = max(0, t0 - window + 1)
        yield t0, t1, b0


def forward(q, k, v, c, g, doc, window: int = 112, scale: Optional[float] = None,
            block: int = 128, return_maps: bool = False):
    """O[T,H,d] (float64).  With return_maps, also the per-block list of
    (t0, t1, b0, P [H, t1-t0, t1-b0], Pbar [t1-t0, t1-b0]) for invariant tests."""
    q, k, v, c, g = map(_f64, (q, k, v, c, g))
    doc = np.asarray(doc)
    T, H, d = q.shape
    sigma = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = np.zeros((T, H, d))
    maps = []
    for t0, t1, b0 in _blocks(T, window, block):
        mask = admitted(doc, np.arange(t0, t1), np.arange(b0, t1), window)
        P = np.empty((H, t1 - t0, t1 - b0))
        for h in range(H):
            S = sigma * (q[t0:t1, h, :] @ k[b0:t1, h, :].T)
            P[h] = _masked_softmax_rows(S, mask)
        Pbar = np.einsum("th,hts->ts", c[t0:t1], P)
        for h in range(H):
            o[t0:t1, h, :] = g[t0:t1, h, None] * (Pbar @ v[b0:t1, h, :])
        if return_maps:
            maps.append((t0, t1, b0, P, Pbar))
    return (o, maps) if return_maps else o


def backward(q, k, v, c, g, doc, do, window: int = 112, scale: Optional[float] = None,
             block: int = 128):
    """(dQ, dK, dV [T,H,d], dC, dG [T,H]) in float64."""
    q, k, v, c, g, do = map(_f64, (q, k, v, c, g, do))
    doc = np.asarray(doc)
    T, H, d = q.shape
    sigma = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = np.zeros((T, H, d))
    dk = np.zeros((T, H, d))
    dv = np.zeros((T, H, d))
    dc = np.zeros((T, H))
    dg = np.zeros((T, H))
    for t0, t1, b0 in _blocks(T, window, block):
        mask = admitted(doc, np.arange(t0, t1), np.arange(b0, t1), window)
        n = t1 - t0
        P = np.empty((H, n, t1 - b0))
        for h in range(H):
            S = sigma * (q[t0:t1, h, :] @ k[b0:t1, h, :].T)
            P[h] = _masked_softmax_rows(S, mask)
        Pbar = np.einsum("th,hts->ts", c[t0:t1], P)
        dPbar = np.zeros((n, t1 - b0))
        for h in range(H):
            A = Pbar @ v[b0:t1, h, :]
            dg[t0:t1, h] = np.sum(do[t0:t1, h, :] * A, axis=-1)
            B = do[t0:t1, h, :] @ v[b0:t1, h, :].T
            dPbar += g[t0:t1, h, None] * B
            dv[b0:t1, h, :] += (g[t0:t1, h, None] * Pbar).T @ do[t0:t1, h, :]
        for h in range(H):
            dc[t0:t1, h] = np.sum(P[h] * dPbar, axis=-1)
            dS = c[t0:t1, h, None] * P[h] * (dPbar - dc[t0:t1, h, None])
            dq[t0:t1, h, :] = sigma * (dS @ k[b0:t1, h, :])
            dk[b0:t1, h, :] += sigma * (dS.T @ q[t0:t1, h, :])
    return dq, dk, dv, dc, dg


def backward_slice(q, k, v, c, g, doc, do, lo: int, hi: int, window: int = 112,
                   scale: Optional[float] = None):
    """Exact gradients for queries [lo, hi) (dQ, dC, dG) and keys [lo, hi)
    (dK, dV) of a long stream, computed on the sub-stream
    [lo-W+1, hi+W-1) so every contributing query sees its whole window."""
    T = q.shape[0]
    a = max(0, lo - window + 1)
    b = min(T, hi + window - 1)
    sl = slice(a, b)
    dq, dk, dv, dc, dg = backward(q[sl], k[sl], v[sl], c[sl], g[sl], doc[sl], do[sl],
                                  window=window, scale=scale)
    r = slice(lo - a, hi - a)
    return dq[r], dk[r], dv[r], dc[r], dg[r]


def forward_slice(q, k, v, c, g, doc, lo: int, hi: int, window: int = 112,
                  scale: Optional[float] = None):
    """Exact O for queries [lo, hi) of a long stream."""
    a = max(0, lo - window + 1)
    sl = slice(a, hi)
    o = forward(q[sl], k[sl], v[sl], c[sl], g[sl], doc[sl], window=window, scale=scale)
    return o[lo - a:]
