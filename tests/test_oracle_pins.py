"""Pins of the fp64 CPU oracle against things other than itself.

Each test below ties the oracle to an independent fact: a hand-worked example,
a dense brute force built a different way, torch.autograd, finite differences,
torch's own attention routine, closed forms and invariants of the layer's
definition (AITNT page "一个国产AI小透明，连续两次刷新NanoGPT Speedrun世界纪录",
section "第二刀-砍层内", Lightweight DC paragraph; readings in oracle/ldc_oracle.py).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import bruteforce as bf
from oracle import ldc_oracle as orc

HERE = os.path.dirname(os.path.abspath(__file__))


def rand_case(seed, T, H, d, ndocs=3, shuffle_ids=False, c_scale=0.7):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, d))
    c = c_scale * rng.standard_normal((T, H))
    g = rng.uniform(0.2, 1.8, (T, H))
    do = rng.standard_normal((T, H, d))
    cuts = np.sort(rng.choice(np.arange(1, max(2, T)), size=min(ndocs - 1, max(0, T - 1)), replace=False))
    doc = np.zeros(T, dtype=np.int32)
    for x in cuts:
        doc[x:] += 1
    if shuffle_ids:  # arbitrary labels: only equality matters
        labels = rng.permutation(1000)[: doc.max() + 1]
        doc = labels[doc].astype(np.int32)
    return q, k, v, c, g, doc, do


# ---------------------------------------------------------------------------
# hand-worked example
# ---------------------------------------------------------------------------
def _ev(x):
    if isinstance(x, (int, float)):
        return float(x)
    return float(eval(x, {"__builtins__": {}}, {"L2": math.log(2), "L3": math.log(3), "ln": math.log}))


def load_golden():
    with open(os.path.join(HERE, "golden", "hand_worked_T5.json")) as f:
        gd = json.load(f)
    arr = lambda key, shape: np.array([[_ev(x) for x in row] for row in gd[key]]).reshape(shape)
    T, H, d = gd["T"], gd["H"], gd["d"]
    ins = dict(q=arr("q", (T, H, d)), k=arr("k", (T, H, d)), v=arr("v", (T, H, d)),
               c=arr("c", (T, H)), g=arr("g", (T, H)), doc=np.array(gd["doc"], dtype=np.int32),
               do=arr("do", (T, H, d)))
    exp = {key: np.array([[_ev(x) for x in row] for row in val]) for key, val in gd["expected"].items()}
    return gd, ins, exp


def test_golden_forward():
    gd, x, e = load_golden()
    o = orc.forward(x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"], window=gd["window"], scale=gd["scale"])
    np.testing.assert_allclose(o[:, :, 0], e["o"], rtol=0, atol=1e-12)


def test_golden_backward():
    gd, x, e = load_golden()
    dq, dk, dv, dc, dg = orc.backward(x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"], x["do"],
                                      window=gd["window"], scale=gd["scale"])
    np.testing.assert_allclose(dg, e["dg"], atol=1e-12)
    np.testing.assert_allclose(dc, e["dc"], atol=1e-12)
    np.testing.assert_allclose(dv[:, :, 0], e["dv"], atol=1e-12)
    np.testing.assert_allclose(dq[:, :, 0], e["dq"], atol=1e-12)
    np.testing.assert_allclose(dk[:, :, 0], e["dk"], atol=1e-12)


# ---------------------------------------------------------------------------
# dense brute force and torch.autograd
# ---------------------------------------------------------------------------
SHAPES = [  # (seed, T, H, d, window, ndocs, block)
    (0, 1, 1, 2, 112, 1, 128),
    (1, 7, 2, 3, 3, 2, 2),
    (2, 40, 3, 4, 5, 3, 7),
    (3, 130, 2, 8, 112, 4, 128),
    (4, 200, 1, 4, 17, 6, 16),
    (5, 150, 2, 2, 300, 2, 64),   # window longer than the stream
    (6, 64, 2, 4, 1, 3, 128),     # window of one key
]


@pytest.mark.parametrize("seed,T,H,d,W,ndocs,block", SHAPES)
def test_forward_matches_bruteforce(seed, T, H, d, W, ndocs, block):
    q, k, v, c, g, doc, _ = rand_case(seed, T, H, d, ndocs, shuffle_ids=(seed % 2 == 1))
    o = orc.forward(q, k, v, c, g, doc, window=W, block=block)
    mask = bf.dense_mask(doc, W)
    ref = bf.forward(*(bf.as_t(x) for x in (q, k, v, c, g)), mask).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed,T,H,d,W,ndocs,block", SHAPES)
def test_backward_matches_autograd(seed, T, H, d, W, ndocs, block):
    q, k, v, c, g, doc, do = rand_case(seed, T, H, d, ndocs)
    grads = orc.backward(q, k, v, c, g, doc, do, window=W, block=block)
    ts = [bf.as_t(x, requires_grad=True) for x in (q, k, v, c, g)]
    out = bf.forward(*ts, bf.dense_mask(doc, W))
    out.backward(bf.as_t(do))
    ref = [t.grad.numpy() for t in ts]  # dq, dk, dv, dc, dg
    for name, a, b in zip(("dq", "dk", "dv", "dc", "dg"), grads, ref):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-10, err_msg=name)


def test_backward_finite_differences():
    """Directional derivatives of the oracle's own forward (central
    differences) against the oracle's backward."""
    q, k, v, c, g, doc, do = rand_case(11, 24, 2, 4, 3)
    W = 5
    grads = orc.backward(q, k, v, c, g, doc, do, window=W)
    rng = np.random.default_rng(12)
    base = [q, k, v, c, g]
    for i, name in enumerate(("q", "k", "v", "c", "g")):
        X = rng.standard_normal(base[i].shape)
        eps = 1e-6

        def L(sign):
            args = list(base)
            args[i] = base[i] + sign * eps * X
            return np.sum(do * orc.forward(*args, doc, window=W))

        fd = (L(+1) - L(-1)) / (2 * eps)
        an = np.sum(grads[i] * X)
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


# ---------------------------------------------------------------------------
# special cases that reduce to library routines or closed forms
# ---------------------------------------------------------------------------
def test_onehot_composition_is_windowed_attention():
    """C = one-hot(h*), G = 1: every head's output is head h*'s softmax map
    applied to that head's values; torch's scaled_dot_product_attention with a
    boolean window mask computes the same thing."""
    T, H, d, W = 160, 3, 8, 37
    q, k, v, c, g, doc, _ = rand_case(21, T, H, d, 4)
    hstar = 1
    c = np.zeros((T, H))
    c[:, hstar] = 1.0
    g = np.ones((T, H))
    o = orc.forward(q, k, v, c, g, doc, window=W)
    t = np.arange(T)
    mask = (t[None, :] <= t[:, None]) & (t[:, None] - t[None, :] < W) & (doc[None, :] == doc[:, None])
    mask_t = torch.from_numpy(mask)
    qh = torch.from_numpy(q[:, hstar, :])[None]
    kh = torch.from_numpy(k[:, hstar, :])[None]
    for h in range(H):
        vh = torch.from_numpy(v[:, h, :])[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask_t)[0].numpy()
        np.testing.assert_allclose(o[:, h, :], ref, rtol=1e-11, atol=1e-11)


def test_constant_values_pass_through():
    """G = 1, sum_h C[t,h] = 1, V[s,h] = v_h for every s: O[t,h] = v_h."""
    T, H, d = 300, 4, 8
    q, k, _, c, _, doc, _ = rand_case(31, T, H, d, 5)
    c = c - c.mean(axis=1, keepdims=True) + 1.0 / H  # rows sum to 1, mixed signs
    vh = np.random.default_rng(32).standard_normal((H, d))
    v = np.broadcast_to(vh[None], (T, H, d)).copy()
    o = orc.forward(q, k, v, c, np.ones((T, H)), doc, window=112)
    np.testing.assert_allclose(o, np.broadcast_to(vh[None], (T, H, d)), atol=1e-12)


def test_window_one_closed_form():
    T, H, d = 90, 3, 4
    q, k, v, c, g, doc, do = rand_case(41, T, H, d, 3)
    o = orc.forward(q, k, v, c, g, doc, window=1)
    np.testing.assert_allclose(o, g[:, :, None] * c.sum(1)[:, None, None] * v, atol=1e-12)
    dq, dk, dv, dc, dg = orc.backward(q, k, v, c, g, doc, do, window=1)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_allclose(dv, g[:, :, None] * c.sum(1)[:, None, None] * do, atol=1e-12)
    dpbar = np.sum(g[:, :, None] * do * v, axis=(1, 2))
    np.testing.assert_allclose(dc, np.broadcast_to(dpbar[:, None], (T, H)), atol=1e-12)


def test_document_start_closed_form():
    T, H, d = 200, 2, 8
    q, k, v, c, g, doc, do = rand_case(51, T, H, d, 6)
    o = orc.forward(q, k, v, c, g, doc)
    dq, *_ = orc.backward(q, k, v, c, g, doc, do)
    starts = np.nonzero(np.r_[True, doc[1:] != doc[:-1]])[0]
    for t in starts:
        np.testing.assert_allclose(o[t], g[t][:, None] * c[t].sum() * v[t], atol=1e-12)
        assert np.all(dq[t] == 0)


def test_row_sums():
    T, H, d = 260, 3, 4
    q, k, v, c, g, doc, _ = rand_case(61, T, H, d, 4)
    _, maps = orc.forward(q, k, v, c, g, doc, return_maps=True)
    for t0, t1, b0, P, Pbar in maps:
        np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-12)
        np.testing.assert_allclose(Pbar.sum(-1), c[t0:t1].sum(1), atol=1e-12)
        assert np.all(P >= 0)


def test_linearity_in_c_and_g():
    T, H, d = 150, 3, 4
    q, k, v, c1, g, doc, _ = rand_case(71, T, H, d, 3)
    c2 = np.random.default_rng(72).standard_normal((T, H))
    f = lambda c, g: orc.forward(q, k, v, c, g, doc)
    np.testing.assert_allclose(f(c1 + 2.5 * c2, g), f(c1, g) + 2.5 * f(c2, g), atol=1e-11)
    g2 = np.random.default_rng(73).uniform(0, 2, (T, H))
    np.testing.assert_allclose(f(c1, g * g2), g2[:, :, None] * f(c1, g), atol=1e-11)


def test_key_shift_invariance():
    T, H, d = 150, 2, 4
    q, k, v, c, g, doc, _ = rand_case(81, T, H, d, 3)
    shift = np.random.default_rng(82).standard_normal((1, H, d))
    np.testing.assert_allclose(orc.forward(q, k + shift, v, c, g, doc),
                               orc.forward(q, k, v, c, g, doc), atol=1e-11)


def test_document_permutation_equivariance():
    T, H, d = 240, 2, 4
    q, k, v, c, g, doc, do = rand_case(91, T, H, d, 5)
    ids = np.unique(doc)
    order = np.random.default_rng(92).permutation(ids)
    perm = np.concatenate([np.nonzero(doc == i)[0] for i in order])
    o = orc.forward(q, k, v, c, g, doc)
    op = orc.forward(q[perm], k[perm], v[perm], c[perm], g[perm], doc[perm])
    np.testing.assert_allclose(op, o[perm], atol=1e-12)
    gr = orc.backward(q, k, v, c, g, doc, do)
    grp = orc.backward(q[perm], k[perm], v[perm], c[perm], g[perm], doc[perm], do[perm])
    for a, b in zip(grp, gr):
        np.testing.assert_allclose(a, b[perm], atol=1e-11)


def test_backward_invariants():
    T, H, d = 300, 3, 8
    q, k, v, c, g, doc, do = rand_case(101, T, H, d, 4)
    o = orc.forward(q, k, v, c, g, doc)
    dq, dk, dv, dc, dg = orc.backward(q, k, v, c, g, doc, do)
    # per token: sum_h C dC = sum_h G dG (both are sum_s Pbar dPbar)
    np.testing.assert_allclose((c * dc).sum(1), (g * dg).sum(1), atol=1e-10)
    # per (t,h): G dG = <dO, O>
    np.testing.assert_allclose(g * dg, np.sum(do * o, axis=-1), atol=1e-10)
    for i in np.unique(doc):
        sel = doc == i
        np.testing.assert_allclose(dk[sel].sum(0), 0.0, atol=1e-10)
        ref = (g[sel][:, :, None] * c[sel].sum(1)[:, None, None] * do[sel]).sum(0)
        np.testing.assert_allclose(dv[sel].sum(0), ref, atol=1e-10)


def test_slices_match_full_stream():
    T, H, d, W = 700, 2, 4, 112
    q, k, v, c, g, doc, do = rand_case(111, T, H, d, 4)
    full = orc.backward(q, k, v, c, g, doc, do, window=W)
    o = orc.forward(q, k, v, c, g, doc, window=W)
    for lo, hi in ((0, 100), (250, 420), (600, 700)):
        sl = orc.backward_slice(q, k, v, c, g, doc, do, lo, hi, window=W)
        for a, b in zip(sl, full):
            np.testing.assert_allclose(a, b[lo:hi], atol=1e-11)
        np.testing.assert_allclose(orc.forward_slice(q, k, v, c, g, doc, lo, hi, window=W), o[lo:hi], atol=1e-12)


def test_block_size_does_not_matter():
    T, H, d = 333, 2, 4
    q, k, v, c, g, doc, do = rand_case(121, T, H, d, 3)
    a = orc.backward(q, k, v, c, g, doc, do, block=128)
    b = orc.backward(q, k, v, c, g, doc, do, block=1)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, atol=1e-11)
