"""Pins of the fp64 DCMHA oracle (oracle/dcmha_oracle.py) against things other
than itself: the independently written Lightweight DC oracle (which DCMHA
reduces to when every head's weight-composition row is G[t,h] C[t,:] and the
score composition is the identity), torch's own attention routine (identity
compositions give plain windowed multi-head attention; permutation matrices
pick other heads' maps), a dense brute force differentiated by
torch.autograd, central finite differences, closed forms and invariants.

Definition: AITNT page "一个国产AI小透明，连续两次刷新NanoGPT Speedrun世界纪录",
section "第二刀-砍层内", DCMHA paragraph (a Compose module transforms attention
scores and weights across heads, dynamically); readings in the oracle's header.
"""
import math

import numpy as np
import pytest
import torch

from oracle import dcmha_oracle as dco
from oracle import ldc_oracle as ldo


def rand_case(seed, T, H, d, ndocs=3, comp_scale=0.6):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, d))
    cs = np.eye(H)[None] + comp_scale * rng.standard_normal((T, H, H))
    cw = comp_scale * rng.standard_normal((T, H, H))
    do = rng.standard_normal((T, H, d))
    cuts = np.sort(rng.choice(np.arange(1, max(2, T)), size=min(ndocs - 1, max(0, T - 1)), replace=False))
    doc = np.zeros(T, dtype=np.int32)
    for x in cuts:
        doc[x:] += 1
    return q, k, v, cs, cw, doc, do


def window_mask(doc, W):
    t = np.arange(len(doc))
    return (t[None, :] <= t[:, None]) & (t[:, None] - t[None, :] < W) & (doc[None, :] == doc[:, None])


# ---------------------------------------------------------------------------
# reductions to independently computed layers
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed,T,H,d,W", [(1, 90, 3, 8, 112), (2, 150, 4, 16, 23), (3, 60, 1, 8, 5)])
def test_reduces_to_lightweight_dc(seed, T, H, d, W):
    """CS = I and CW[t,h,:] = G[t,h] C[t,:] (every head's row is the shared
    composition C, scaled by the head scale): DCMHA is the Lightweight DC layer.
    Its gradients map through the chain rule: dC[t,h'] = sum_h G[t,h] dCW[t,h,h'],
    dG[t,h] = sum_h' C[t,h'] dCW[t,h,h']."""
    q, k, v, _, _, doc, do = rand_case(seed, T, H, d)
    rng = np.random.default_rng(seed + 100)
    c = 0.7 * rng.standard_normal((T, H))
    g = rng.uniform(0.2, 1.8, (T, H))
    cs = np.broadcast_to(np.eye(H)[None], (T, H, H)).copy()
    cw = g[:, :, None] * c[:, None, :]
    o = dco.forward(q, k, v, cs, cw, doc, window=W)
    np.testing.assert_allclose(o, ldo.forward(q, k, v, c, g, doc, window=W), rtol=1e-11, atol=1e-12)
    dq, dk, dv, dcs, dcw = dco.backward(q, k, v, cs, cw, doc, do, window=W)
    rq, rk, rv, rc, rg = ldo.backward(q, k, v, c, g, doc, do, window=W)
    for a, b in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(np.einsum("th,thg->tg", g, dcw), rc, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(np.einsum("tg,thg->th", c, dcw), rg, rtol=1e-10, atol=1e-11)


def _sdpa_heads(q, k, v, mask, src):
    """Per head h: softmax attention of head src[h]'s Q, K applied to head h's V
    (torch's scaled_dot_product_attention with a boolean mask)."""
    T, H, d = q.shape
    m = torch.from_numpy(mask)
    out = np.zeros((T, H, d))
    for h in range(H):
        qh = torch.from_numpy(q[:, src[h], :])[None]
        kh = torch.from_numpy(k[:, src[h], :])[None]
        vh = torch.from_numpy(v[:, h, :])[None]
        out[:, h, :] = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, attn_mask=m)[0].numpy()
    return out


def test_identity_is_windowed_multihead_attention():
    """CS = CW = I: plain per-head softmax attention over the window."""
    T, H, d, W = 140, 3, 8, 37
    q, k, v, _, _, doc, _ = rand_case(11, T, H, d, 4)
    eye = np.broadcast_to(np.eye(H)[None], (T, H, H)).copy()
    o = dco.forward(q, k, v, eye, eye, doc, window=W)
    np.testing.assert_allclose(o, _sdpa_heads(q, k, v, window_mask(doc, W), list(range(H))),
                               rtol=1e-11, atol=1e-11)


def test_identity_backward_matches_sdpa_autograd():
    """CS = CW = I: dQ, dK, dV equal torch.autograd through torch's attention
    routine (fp64)."""
    T, H, d, W = 70, 2, 8, 19
    q, k, v, _, _, doc, do = rand_case(12, T, H, d, 3)
    eye = np.broadcast_to(np.eye(H)[None], (T, H, H)).copy()
    dq, dk, dv, _, _ = dco.backward(q, k, v, eye, eye, doc, do, window=W)
    m = torch.from_numpy(window_mask(doc, W))
    tq, tk, tv = (torch.from_numpy(x.transpose(1, 0, 2).copy()).requires_grad_(True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m)
    out.backward(torch.from_numpy(do.transpose(1, 0, 2).copy()))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy().transpose(1, 0, 2), rtol=1e-10, atol=1e-11)


def test_permutations_pick_other_heads():
    """CS = perm a, CW = perm b (row h has its 1 at column a[h], b[h]): head h's
    output is head a[b[h]]'s attention map applied to head h's values.  A
    transposed matrix or a swapped index fails this."""
    T, H, d, W = 120, 4, 8, 50
    q, k, v, _, _, doc, _ = rand_case(13, T, H, d, 3)
    a, b = [2, 0, 3, 1], [1, 3, 0, 2]
    cs = np.zeros((T, H, H))
    cw = np.zeros((T, H, H))
    for h in range(H):
        cs[:, h, a[h]] = 1.0
        cw[:, h, b[h]] = 1.0
    o = dco.forward(q, k, v, cs, cw, doc, window=W)
    np.testing.assert_allclose(o, _sdpa_heads(q, k, v, window_mask(doc, W), [a[b[h]] for h in range(H)]),
                               rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------------------------
# a dense brute force and torch.autograd
# ---------------------------------------------------------------------------
def dense_forward(q, k, v, cs, cw, mask, scale):
    """All T x T maps at once; masked scores -inf before the softmax."""
    S = scale * torch.einsum("thj,shj->hts", q, k)
    Z = torch.einsum("tab,bts->ats", cs, S)
    Z = Z.masked_fill(~mask[None], float("-inf"))
    P = torch.softmax(Z, dim=-1)
    R = torch.einsum("tab,bts->ats", cw, P)
    return torch.einsum("hts,shj->thj", R, v)


@pytest.mark.parametrize("seed,T,H,d,W,ndocs", [(21, 40, 3, 4, 112, 2), (22, 64, 2, 8, 9, 5),
                                                  (23, 33, 4, 4, 1, 1)])
def test_matches_dense_autograd(seed, T, H, d, W, ndocs):
    q, k, v, cs, cw, doc, do = rand_case(seed, T, H, d, ndocs)
    mask = torch.zeros(T, T, dtype=torch.bool)
    for t in range(T):  # filled entry by entry, independently of the oracle's gather
        for s in range(T):
            mask[t, s] = bool(s <= t and t - s < W and doc[s] == doc[t])
    xs = [torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v, cs, cw)]
    out = dense_forward(*xs, mask, 1.0 / math.sqrt(d))
    out.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dco.forward(q, k, v, cs, cw, doc, window=W), out.detach().numpy(),
                               rtol=1e-11, atol=1e-12)
    for mine, x in zip(dco.backward(q, k, v, cs, cw, doc, do, window=W), xs):
        np.testing.assert_allclose(mine, x.grad.numpy(), rtol=1e-10, atol=1e-11)


def test_backward_finite_differences():
    """Directional derivatives of L = <dO, O> by central differences, for every input."""
    T, H, d, W = 12, 3, 4, 5
    q, k, v, cs, cw, doc, do = rand_case(31, T, H, d, 2)
    ins = [q, k, v, cs, cw]
    grads = dco.backward(q, k, v, cs, cw, doc, do, window=W)
    rng = np.random.default_rng(32)
    eps = 1e-6
    for i, name in enumerate(("q", "k", "v", "cs", "cw")):
        X = rng.standard_normal(ins[i].shape)

        def L(sign):
            moved = list(ins)
            moved[i] = ins[i] + sign * eps * X
            return np.sum(do * dco.forward(*moved, doc, window=W))

        fd = (L(+1) - L(-1)) / (2 * eps)
        an = np.sum(grads[i] * X)
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


# ---------------------------------------------------------------------------
# closed forms and invariants
# ---------------------------------------------------------------------------
def test_window_one_closed_form():
    """W = 1: the only admitted key is t itself, so every P is 1 whatever CS is;
    O[t,h] = (sum_h' CW[t,h,h']) V[t,h], and no gradient reaches Q, K or CS."""
    T, H, d = 50, 3, 6
    q, k, v, cs, cw, doc, do = rand_case(41, T, H, d, 4)
    o = dco.forward(q, k, v, cs, cw, doc, window=1)
    np.testing.assert_allclose(o, cw.sum(axis=2)[:, :, None] * v, rtol=1e-12, atol=1e-12)
    dq, dk, dv, dcs, dcw = dco.backward(q, k, v, cs, cw, doc, do, window=1)
    for x in (dq, dk, dcs):
        assert np.abs(x).max() < 1e-12
    np.testing.assert_allclose(dv, cw.sum(axis=2)[:, :, None] * do, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dcw, np.einsum("thj,thj->th", do, v)[:, :, None] * np.ones((1, 1, H)),
                               rtol=1e-12, atol=1e-12)


def test_constant_values_pass_through():
    """CW rows summing to 1 and V[s,h] = v_h for every s: O[t,h] = v_h."""
    T, H, d = 200, 4, 8
    q, k, _, cs, cw, doc, _ = rand_case(42, T, H, d, 5)
    cw = cw - cw.mean(axis=2, keepdims=True) + 1.0 / H
    vh = np.random.default_rng(43).standard_normal((H, d))
    o = dco.forward(q, k, np.broadcast_to(vh[None], (T, H, d)).copy(), cs, cw, doc, window=112)
    np.testing.assert_allclose(o, np.broadcast_to(vh[None], (T, H, d)), atol=1e-12)


def test_homogeneity_identities():
    """O is linear in V and in CW, and scaling CS is scaling the scores, i.e. Q
    (or K): so <dV,V> = <dCW,CW> = <dO,O> and <dCS,CS> = <dQ,Q> = <dK,K>."""
    T, H, d, W = 160, 3, 8, 112
    q, k, v, cs, cw, doc, do = rand_case(44, T, H, d, 3)
    o = dco.forward(q, k, v, cs, cw, doc, window=W)
    dq, dk, dv, dcs, dcw = dco.backward(q, k, v, cs, cw, doc, do, window=W)
    ref = np.sum(do * o)
    assert np.isclose(np.sum(dv * v), ref, rtol=1e-11)
    assert np.isclose(np.sum(dcw * cw), ref, rtol=1e-11)
    sq = np.sum(dq * q)
    assert np.isclose(np.sum(dcs * cs), sq, rtol=1e-10)
    assert np.isclose(np.sum(dk * k), sq, rtol=1e-10)


def test_causal_and_document_cut():
    """Changing a key/value at a later position or in another document changes no output row."""
    T, H, d, W = 90, 2, 4, 30
    q, k, v, cs, cw, doc, _ = rand_case(45, T, H, d, 3)
    o = dco.forward(q, k, v, cs, cw, doc, window=W)
    k2, v2 = k.copy(), v.copy()
    t0 = 60
    k2[t0 + 1:] += 5.0
    v2[t0 + 1:] -= 3.0
    o2 = dco.forward(q, k2, v2, cs, cw, doc, window=W)
    np.testing.assert_array_equal(o[: t0 + 1], o2[: t0 + 1])
    other = doc != doc[t0]
    k3, v3 = k.copy(), v.copy()
    k3[other] = 7.0
    v3[other] = -2.0
    o3 = dco.forward(q, k3, v3, cs, cw, doc, window=W)
    np.testing.assert_array_equal(o[doc == doc[t0]], o3[doc == doc[t0]])
