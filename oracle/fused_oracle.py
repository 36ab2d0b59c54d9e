"""Plain fp64 CPU oracle of the Lightweight DC layer fused with the attention
block's main attention.

TEST INFRASTRUCTURE.  Only tests, the smoke check and the CPU-baseline leg of
the benchmark may import this module.  It shares no code with the HIP path and
imports nothing from it.

What is computed (AITNT page "一个国产AI小透明，连续两次刷新NanoGPT
Speedrun世界纪录", section "第二刀-砍层内", Lightweight DC paragraph: the branch
reuses the attention block's Q and K, works on a short local window, and keeps
its overhead down with a dedicated kernel).  The page does not give the main
attention's form or how the two outputs meet; the readings taken:

* F1 the main attention is causal softmax attention of every head over the
  query's own document, a document being a contiguous run of equal ids:
  key s is admitted for query t iff run_start(t) <= s <= t, where run_start(t)
  is the first token of the run that holds t;
* F2 the block's output is the sum of the main attention's and the Lightweight
  DC layer's outputs, the latter exactly as in ldc_oracle (same Q, K, V, its
  own window and document rule, C and G);
* F3 both use the same softmax scale (1/sqrt(d) unless given).

    run_start(t) = max{ s <= t : s == 0 or doc[s] != doc[s-1] }
    M[t,h]       = sum_{s = run_start(t)}^{t} softmax_s(sigma <Q[t,h], K[s,h]>) V[s,h]
    O[t,h]       = M[t,h] + LDC(Q, K, V, C, G, doc)[t,h]

Each query is evaluated on its own in float64 (numpy), heads together.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import ldc_oracle


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def run_start(doc) -> np.ndarray:
    """int64 [T]: the first token of the contiguous run of equal ids holding t."""
    doc = np.asarray(doc)
    T = doc.shape[0]
    out = np.zeros(T, dtype=np.int64)
    start = 0
    for t in range(T):
        if t > 0 and doc[t] != doc[t - 1]:
            start = t
        out[t] = start
    return out


def main_attention(q, k, v, doc, scale: Optional[float] = None, queries=None) -> np.ndarray:
    """M[T,H,d] (float64), or only the rows of `queries` (in that order)."""
    q, k, v = map(_f64, (q, k, v))
    T, H, d = q.shape
    sigma = 1.0 / np.sqrt(d) if scale is None else float(scale)
    rs = run_start(doc)
    ts = range(T) if queries is None else queries
    out = np.zeros((len(ts), H, d))
    for row, t in enumerate(ts):
        lo = rs[t]
        kk, vv = k[lo:t + 1], v[lo:t + 1]            # [n, H, d]
        s = sigma * np.einsum("hd,nhd->hn", q[t], kk)  # [H, n]
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        p = e / e.sum(axis=1, keepdims=True)
        out[row] = np.einsum("hn,nhd->hd", p, vv)
    return out


def forward(q, k, v, c, g, doc, window: int = 112, scale: Optional[float] = None) -> np.ndarray:
    """O[T,H,d] (float64): main attention plus the Lightweight DC layer."""
    return main_attention(q, k, v, doc, scale) + ldc_oracle.forward(q, k, v, c, g, doc, window, scale)


def forward_rows(q, k, v, c, g, doc, queries, window: int = 112, scale: Optional[float] = None) -> np.ndarray:
    """O for the given query rows of a long stream (each with its whole run and window)."""
    queries = list(queries)
    m = main_attention(q, k, v, doc, scale, queries)
    out = np.zeros_like(m)
    for row, t in enumerate(queries):
        out[row] = m[row] + ldc_oracle.forward_slice(q, k, v, c, g, doc, t, t + 1, window, scale)[0]
    return out
