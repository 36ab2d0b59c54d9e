"""Pins of the MUDD mixing oracle against facts fixed by the definition itself
(AITNT page "一个国产AI小透明，连续两次刷新NanoGPT Speedrun世界纪录", section
"第一刀—砍层间"): scalar brute force on tiny inputs, selection by one-hot
weights, affine combinations of equal streams, the bilinear adjoint
identities, and central finite differences.  CPU only."""
import numpy as np
import pytest

from oracle import mudd_oracle as mo


def rand_case(rng, T=5, dm=7, W=3, J=4):
    xs = [rng.standard_normal((T, dm)) for _ in range(J)]
    a = rng.standard_normal((T, W, J))
    dys = [rng.standard_normal((T, dm)) for _ in range(W)]
    return xs, a, dys


def brute_forward(xs, a):
    T, dm = len(xs[0]), len(xs[0][0])
    W, J = len(a[0]), len(xs)
    y = [[[0.0] * dm for _ in range(T)] for _ in range(W)]
    for w in range(W):
        for t in range(T):
            for c in range(dm):
                s = 0.0
                for j in range(J):
                    s += float(a[t][w][j]) * float(xs[j][t][c])
                y[w][t][c] = s
    return np.array(y)


def brute_backward(xs, a, dys):
    T, dm = len(xs[0]), len(xs[0][0])
    W, J = len(a[0]), len(xs)
    dx = [[[0.0] * dm for _ in range(T)] for _ in range(J)]
    da = [[[0.0] * J for _ in range(W)] for _ in range(T)]
    for t in range(T):
        for j in range(J):
            for c in range(dm):
                dx[j][t][c] = sum(float(a[t][w][j]) * float(dys[w][t][c]) for w in range(W))
            for w in range(W):
                da[t][w][j] = sum(float(dys[w][t][c]) * float(xs[j][t][c]) for c in range(dm))
    return np.array(dx), np.array(da)


@pytest.mark.parametrize("shape", [(1, 1, 1, 1), (3, 5, 1, 2), (4, 6, 4, 3), (2, 9, 2, 5)])
def test_brute_force(shape):
    T, dm, W, J = shape
    xs, a, dys = rand_case(np.random.default_rng(sum(shape)), T, dm, W, J)
    np.testing.assert_allclose(mo.forward(xs, a), brute_forward(xs, a), rtol=1e-13, atol=1e-13)
    dx, da = mo.backward(xs, a, dys)
    bdx, bda = brute_backward(xs, a, dys)
    np.testing.assert_allclose(dx, bdx, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(da, bda, rtol=1e-13, atol=1e-13)


def test_one_hot_weights_select_a_stream():
    rng = np.random.default_rng(1)
    T, dm, W, J = 6, 8, 4, 5
    xs, _, _ = rand_case(rng, T, dm, W, J)
    sel = rng.integers(0, J, size=(T, W))
    a = np.zeros((T, W, J))
    for t in range(T):
        for w in range(W):
            a[t, w, sel[t, w]] = 1.0
    y = mo.forward(xs, a)
    for t in range(T):
        for w in range(W):
            assert np.array_equal(y[w, t], xs[sel[t, w]][t])


def test_affine_mix_of_equal_streams_is_the_stream():
    rng = np.random.default_rng(2)
    T, dm, W, J = 5, 6, 2, 4
    x = rng.standard_normal((T, dm))
    a = rng.standard_normal((T, W, J))
    a[:, :, -1] = 1.0 - a[:, :, :-1].sum(axis=2)  # weights of each (t, w) sum to 1, signs mixed
    y = mo.forward([x] * J, a)
    for w in range(W):
        np.testing.assert_allclose(y[w], x, rtol=0, atol=1e-12)


def test_single_stream_single_way_is_a_row_scale():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((7, 3))
    a = rng.standard_normal((7, 1, 1))
    np.testing.assert_allclose(mo.forward([x], a)[0], a[:, 0, 0][:, None] * x, rtol=1e-15, atol=0)
    dy = rng.standard_normal((7, 3))
    dx, da = mo.backward([x], a, [dy])
    np.testing.assert_allclose(dx[0], a[:, 0, 0][:, None] * dy, rtol=1e-15, atol=0)
    np.testing.assert_allclose(da[:, 0, 0], (x * dy).sum(axis=1), rtol=1e-13, atol=0)


def test_zero_weights_give_zero_output_and_input_gradient():
    rng = np.random.default_rng(4)
    xs, a, dys = rand_case(rng)
    a[:] = 0.0
    assert not mo.forward(xs, a).any()
    dx, da = mo.backward(xs, a, dys)
    assert not dx.any() and da.any()


def test_adjoint_identities():
    # L = sum_w <dY_w, Y_w> is bilinear: L = sum_j <X_j, dX_j> = sum a * dA
    xs, a, dys = rand_case(np.random.default_rng(5), T=6, dm=11, W=4, J=3)
    y = mo.forward(xs, a)
    dx, da = mo.backward(xs, a, dys)
    L = sum(float(np.sum(dys[w] * y[w])) for w in range(len(dys)))
    assert abs(L - sum(float(np.sum(xs[j] * dx[j])) for j in range(len(xs)))) < 1e-10 * (1 + abs(L))
    assert abs(L - float(np.sum(a * da))) < 1e-10 * (1 + abs(L))


def test_finite_differences():
    rng = np.random.default_rng(6)
    xs, a, dys = rand_case(rng, T=3, dm=4, W=2, J=3)
    dx, da = mo.backward(xs, a, dys)

    def loss(xs_, a_):
        y = mo.forward(xs_, a_)
        return sum(float(np.sum(dys[w] * y[w])) for w in range(len(dys)))

    h = 1e-6
    for (t, w, j) in [(0, 0, 0), (1, 1, 2), (2, 0, 1)]:
        ap, am = a.copy(), a.copy()
        ap[t, w, j] += h
        am[t, w, j] -= h
        assert abs((loss(xs, ap) - loss(xs, am)) / (2 * h) - da[t, w, j]) < 1e-7
    for (j, t, c) in [(0, 0, 0), (2, 1, 3), (1, 2, 1)]:
        xp = [x.copy() for x in xs]
        xm = [x.copy() for x in xs]
        xp[j][t, c] += h
        xm[j][t, c] -= h
        assert abs((loss(xp, a) - loss(xm, a)) / (2 * h) - dx[j, t, c]) < 1e-7


def test_shape_errors():
    rng = np.random.default_rng(7)
    xs, a, dys = rand_case(rng)
    with pytest.raises(ValueError):
        mo.forward(xs[:-1], a)
    with pytest.raises(ValueError):
        mo.backward(xs, a, dys[:-1])
