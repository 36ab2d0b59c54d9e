"""Pins of the fp64 generator oracle (oracle/cg_oracle.py): elementwise sums
written as Python loops on tiny inputs, one-hot inputs that select rows and
columns, linearity, the adjoint identity, finite differences and torch
autograd.  Reading in the oracle's header (AITNT page, section "第二刀-砍层内")."""
import numpy as np
import torch

from oracle import cg_oracle as cgo


def case(seed, T=13, dm=10, H=3):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, dm)), rng.standard_normal((dm, H)), rng.standard_normal((dm, H)),
            rng.standard_normal((T, H)), rng.standard_normal((T, H)))


def test_loops_on_tiny_inputs():
    x, wc, wg, dc, dg = case(1, T=4, dm=5, H=2)
    c, g = cgo.forward(x, wc, wg)
    dx, dwc, dwg = cgo.backward(x, wc, wg, dc, dg)
    for t in range(4):
        for h in range(2):
            assert np.isclose(c[t, h], sum(x[t, i] * wc[i, h] for i in range(5)), rtol=1e-14)
            assert np.isclose(g[t, h], sum(x[t, i] * wg[i, h] for i in range(5)), rtol=1e-14)
        for i in range(5):
            ref = sum(dc[t, h] * wc[i, h] + dg[t, h] * wg[i, h] for h in range(2))
            assert np.isclose(dx[t, i], ref, rtol=1e-13, atol=1e-14)
    for i in range(5):
        for h in range(2):
            assert np.isclose(dwc[i, h], sum(x[t, i] * dc[t, h] for t in range(4)), rtol=1e-13, atol=1e-14)
            assert np.isclose(dwg[i, h], sum(x[t, i] * dg[t, h] for t in range(4)), rtol=1e-13, atol=1e-14)


def test_one_hot_inputs_select_rows():
    """x[t] = e_i: C[t] is row i of WC; dC = e_h at one token: dx row is column h of WC."""
    _, wc, wg, _, _ = case(2)
    x = np.zeros((10, 10))
    x[np.arange(10), np.arange(10)[::-1]] = 1.0
    c, g = cgo.forward(x, wc, wg)
    np.testing.assert_array_equal(c, wc[::-1])
    np.testing.assert_array_equal(g, wg[::-1])
    dc = np.zeros((10, 3))
    dc[4, 1] = 1.0
    dx, dwc, dwg = cgo.backward(x, wc, wg, dc, np.zeros((10, 3)))
    np.testing.assert_array_equal(dx[4], wc[:, 1])
    assert np.all(dx[np.arange(10) != 4] == 0)
    assert np.all(dwg == 0)
    np.testing.assert_array_equal(dwc[:, 1], x[4])


def test_adjoint_and_linearity():
    """<dC, x WC> + <dG, x WG> = <dx, x> = <dWC, WC> + <dWG, WG> (bilinearity)."""
    x, wc, wg, dc, dg = case(3, T=50, dm=24, H=6)
    c, g = cgo.forward(x, wc, wg)
    dx, dwc, dwg = cgo.backward(x, wc, wg, dc, dg)
    ref = np.sum(dc * c) + np.sum(dg * g)
    assert np.isclose(np.sum(dx * x), ref, rtol=1e-12)
    assert np.isclose(np.sum(dwc * wc) + np.sum(dwg * wg), ref, rtol=1e-12)
    c2, g2 = cgo.forward(2.5 * x, wc, wg)
    np.testing.assert_allclose(c2, 2.5 * c, rtol=1e-13)
    np.testing.assert_allclose(g2, 2.5 * g, rtol=1e-13)


def test_finite_differences_and_autograd():
    x, wc, wg, dc, dg = case(4)
    grads = cgo.backward(x, wc, wg, dc, dg)
    ins = [x, wc, wg]
    rng = np.random.default_rng(5)
    for i in range(3):
        X = rng.standard_normal(ins[i].shape)

        def L(s):
            moved = list(ins)
            moved[i] = ins[i] + s * 1e-6 * X
            c, g = cgo.forward(*moved)
            return np.sum(dc * c) + np.sum(dg * g)

        fd = (L(1) - L(-1)) / 2e-6
        assert abs(fd - np.sum(grads[i] * X)) <= 1e-7 * max(1.0, abs(fd))
    tx, twc, twg = (torch.from_numpy(a.copy()).requires_grad_(True) for a in ins)
    (torch.sum(torch.from_numpy(dc) * (tx @ twc)) + torch.sum(torch.from_numpy(dg) * (tx @ twg))).backward()
    for mine, t in zip(grads, (tx, twc, twg)):
        np.testing.assert_allclose(mine, t.grad.numpy(), rtol=1e-12, atol=1e-12)
