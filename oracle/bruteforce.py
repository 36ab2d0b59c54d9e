"""Dense brute-force Lightweight DC forward in torch float64 (CPU).

TEST INFRASTRUCTURE, used only to pin the blocked oracle in `ldc_oracle`.  It is
built differently on purpose: the admission mask is a dense T x T matrix filled
one entry at a time by a Python loop over (t, s), the softmax is torch's, and
the backward pass is whatever torch.autograd derives from this forward — no
hand-written gradient.  Only for T up to a few hundred tokens.

Definition followed: AITNT page "一个国产AI小透明，连续两次刷新NanoGPT Speedrun
世界纪录", section "第二刀-砍层内", Lightweight DC paragraph (per-head softmax in
a 112-token local window, post-softmax composition of the heads' maps into one
shared map, per-head scale on each head's Value path), with the readings listed
in `ldc_oracle`.
"""
from __future__ import annotations

import math

import torch


def dense_mask(doc, window: int) -> torch.Tensor:
    T = len(doc)
    m = torch.zeros(T, T, dtype=torch.bool)
    for t in range(T):
        for s in range(T):
            if s <= t and t - s < window and int(doc[s]) == int(doc[t]):
                m[t, s] = True
    return m


def forward(q, k, v, c, g, mask: torch.Tensor, scale=None) -> torch.Tensor:
    """q, k, v: [T,H,d]; c, g: [T,H]; mask: [T,T] bool.  Tensors may require grad."""
    T, H, d = q.shape
    sigma = 1.0 / math.sqrt(d) if scale is None else scale
    S = sigma * torch.einsum("thj,shj->hts", q, k)            # [H,T,T]
    S = S.masked_fill(~mask[None], float("-inf"))
    P = torch.softmax(S, dim=-1)                              # [H,T,T]
    Pbar = (c.transpose(0, 1)[:, :, None] * P).sum(dim=0)     # [T,T]
    A = torch.einsum("ts,shj->thj", Pbar, v)                  # [T,H,d]
    return g[:, :, None] * A


def as_t(x, requires_grad=False) -> torch.Tensor:
    t = torch.as_tensor(x).to(torch.float64).clone()
    t.requires_grad_(requires_grad)
    return t
