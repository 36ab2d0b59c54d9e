"""Pins of the fp64 oracle of the fused block (oracle/fused_oracle.py): the
run starts by brute force; the main attention against torch's own attention
routine under a dense causal run mask, against a brute-force softmax written
with Python loops, against the closed form of a one-token run, and against
the Lightweight DC oracle where every run fits in the window (one-hot C picks
one head's map); the sum with the Lightweight DC layer.

Definition: AITNT page "一个国产AI小透明，连续两次刷新NanoGPT Speedrun世界纪录",
section "第二刀-砍层内", Lightweight DC paragraph (the branch reuses the block's
Q and K); readings F1-F3 in the oracle's header.
"""
import math

import numpy as np
import torch

from oracle import fused_oracle as fo
from oracle import ldc_oracle as ldo


def case(seed, T, H, d, cuts):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((T, H, d)) for _ in range(3))
    c = rng.standard_normal((T, H))
    g = rng.uniform(0, 2, (T, H))
    doc = np.zeros(T, dtype=np.int32)
    for x in cuts:
        doc[x:] += 1
    return q, k, v, c, g, doc


def test_run_start_brute_force():
    rng = np.random.default_rng(0)
    for _ in range(20):
        T = int(rng.integers(1, 60))
        doc = rng.integers(0, 3, T)  # repeated ids in separate runs included
        rs = fo.run_start(doc)
        for t in range(T):
            s = t
            while s > 0 and doc[s - 1] == doc[t]:
                s -= 1
            assert rs[t] == s


def test_main_attention_against_torch_sdpa():
    """Runs with repeated ids (0, 1, 0, 2, 2 as separate runs): a query sees
    only its own run, the run starts found here by walking back."""
    q, k, v, _, _, _ = case(1, 70, 3, 16, [])
    doc = np.array([0] * 9 + [1] * 20 + [0] * 12 + [2] * 1 + [1] * 28, dtype=np.int32)
    rs = np.zeros(70, dtype=np.int64)
    for i in range(70):
        s = i
        while s > 0 and doc[s - 1] == doc[i]:
            s -= 1
        rs[i] = s
    t = np.arange(70)
    mask = (t[None, :] <= t[:, None]) & (t[None, :] >= rs[:, None])
    qt, kt, vt = (torch.from_numpy(x).permute(1, 0, 2) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask))
    np.testing.assert_allclose(fo.main_attention(q, k, v, doc), ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_main_attention_loops_and_scale():
    q, k, v, _, _, doc = case(2, 9, 2, 4, [3, 7])
    rs = fo.run_start(doc)
    got = fo.main_attention(q, k, v, doc, scale=0.7)
    for t in range(9):
        for h in range(2):
            keys = list(range(rs[t], t + 1))
            w = [math.exp(0.7 * sum(q[t, h, j] * k[s, h, j] for j in range(4))) for s in keys]
            z = sum(w)
            for j in range(4):
                assert math.isclose(got[t, h, j], sum(wi * v[s, h, j] for wi, s in zip(w, keys)) / z,
                                    rel_tol=1e-11, abs_tol=1e-12)


def test_one_token_runs_return_own_value():
    """Every token its own document: each query attends only to itself."""
    q, k, v, _, _, _ = case(3, 12, 2, 8, [])
    doc = np.arange(12)
    np.testing.assert_allclose(fo.main_attention(q, k, v, doc), v, rtol=0, atol=1e-15)


def test_short_runs_match_the_lightweight_dc_head_map():
    """Runs no longer than the window: with C one-hot on head h and G = 1 the
    Lightweight DC layer applies head h's windowed attention map to every
    head's V, so its head-h output is the main attention of head h."""
    T, H, d = 200, 3, 8
    q, k, v, _, _, doc = case(4, T, H, d, list(range(37, T, 37)))
    m = fo.main_attention(q, k, v, doc)
    for h in range(H):
        c = np.zeros((T, H))
        c[:, h] = 1.0
        o = ldo.forward(q, k, v, c, np.ones((T, H)), doc, window=112)
        np.testing.assert_allclose(m[:, h], o[:, h], rtol=1e-12, atol=1e-12)


def test_forward_is_main_plus_lightweight_dc():
    q, k, v, c, g, doc = case(5, 150, 2, 8, [60, 61, 100])
    o = fo.forward(q, k, v, c, g, doc, window=20)
    np.testing.assert_allclose(o, fo.main_attention(q, k, v, doc) + ldo.forward(q, k, v, c, g, doc, window=20),
                               rtol=0, atol=0)
    rows = [0, 59, 60, 61, 99, 149]
    np.testing.assert_allclose(fo.forward_rows(q, k, v, c, g, doc, rows, window=20), o[rows], rtol=1e-12,
                               atol=1e-12)
