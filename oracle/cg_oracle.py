"""Plain fp64 CPU oracle of the generator of the Lightweight DC weights.

TEST INFRASTRUCTURE.  Only tests, the smoke check and the CPU-baseline leg of
the benchmark may import this module.  It shares no code with the HIP path and
imports nothing from it.

What is computed (AITNT page "一个国产AI小透明，连续两次刷新NanoGPT
Speedrun世界纪录", section "第二刀-砍层内"): the DCMHA paragraph says the
composition is decided from the current input, and the Lightweight DC
paragraph that the heads' maps are composed dynamically into the shared map
and act on each head's Value through per-head scales.  The page does not give
the generator's form; the reading taken is the plainest one: both weights are
linear projections of the layer's input hidden state x[t] (the row the block's
Q, K, V projections also read), with no bias and no nonlinearity:

    C[t, h] = sum_i x[t, i] WC[i, h]         G[t, h] = sum_i x[t, i] WG[i, h]

Backward, given dC and dG:

    dx[t, i]  = sum_h dC[t, h] WC[i, h] + dG[t, h] WG[i, h]
    dWC[i, h] = sum_t x[t, i] dC[t, h]       dWG[i, h] = sum_t x[t, i] dG[t, h]

Each formula is evaluated as written with float64 numpy products.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def forward(x, wc, wg):
    """(C, G), each [T, H] float64."""
    x, wc, wg = map(_f64, (x, wc, wg))
    return x @ wc, x @ wg


def backward(x, wc, wg, dc, dg):
    """(dx [T, dm], dWC [dm, H], dWG [dm, H]) in float64."""
    x, wc, wg, dc, dg = map(_f64, (x, wc, wg, dc, dg))
    dx = dc @ wc.T + dg @ wg.T
    return dx, x.T @ dc, x.T @ dg
