"""Parity of the HIP MUDD mixing kernels with the fp64 oracle, through the C ABI.

Every output element is an fp32 sum of fp32 products of stored (exact) values,
so both storage dtypes are held to the fp32 bar: relative L2 <= 1e-5 and max
abs error <= 1e-5 x max |reference|, per output tensor."""
import numpy as np
import pytest

from dynamic_head_composition_amd import workloads as wl
from oracle import mudd_oracle as mo

pytestmark = pytest.mark.gpu

TOL = 1e-5


def check(name, got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    scale = max(float(np.max(np.abs(ref))), 1e-30)
    rel = float(np.linalg.norm(got - ref) / max(float(np.linalg.norm(ref)), 1e-30))
    print(f"  {name}: max_abs={err.max():.3e} (scale {scale:.3g}) rel_l2={rel:.3e}", flush=True)
    assert err.max() <= TOL * scale, name
    assert rel <= TOL, name


def run(ldc, w):
    import torch
    from dynamic_head_composition_amd import mudd
    xs, a, dys = w.torch_inputs("cuda")
    ys = mudd.fwd(xs, a)
    dxs, da = mudd.bwd(xs, a, dys)
    torch.cuda.synchronize()
    return ([y.cpu().numpy() for y in ys], [d.cpu().numpy() for d in dxs], da.cpu().numpy())


# (T, dm, W, J, dtype, seed): one-slot and multi-slot rows, partial slots
# (dm % 256 != 0), a row split into two slot groups (dm = 1028: 5 slots), the
# largest dm, every W, J from 1 to the maximum, ragged T.
CASES = [
    (1, 4, 1, 1, "f32", 1),
    (37, 96, 1, 1, "bf16", 2),
    (100, 200, 4, 13, "bf16", 3),
    (64, 768, 4, 13, "bf16", 4),
    (131, 768, 1, 12, "bf16", 5),
    (33, 1028, 2, 5, "f32", 6),
    (19, 4096, 3, 16, "bf16", 7),
    (5, 16384, 1, 2, "f32", 8),
    (257, 512, 4, 3, "f32", 9),
    (6001, 768, 4, 13, "bf16", 10),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T{}_dm{}_W{}_J{}_{}".format(*c[:5]))
def test_parity(ldc, case):
    T, dm, W, J, dtype, seed = case
    print(f"mudd parity case {case}", flush=True)
    w = wl.make_mudd_workload(T, dm, W, J, dtype=dtype, seed=seed)
    ys, dxs, da = run(ldc, w)
    ry = mo.forward(w.xs, w.a)
    rdx, rda = mo.backward(w.xs, w.a, w.dys)
    for k in range(W):
        check(f"y{k}", ys[k], ry[k])
    for j in range(J):
        check(f"dx{j}", dxs[j], rdx[j])
    check("da", da, rda)


def test_full_size_sampled_rows(ldc):
    """The benchmark's workload, in the launch configuration it times, checked
    on sampled rows (each output row depends on its own token only)."""
    cfg = dict(wl.MUDD_BENCH)
    print(f"mudd full-size case {cfg}", flush=True)
    w = wl.make_mudd_workload(**cfg)
    ys, dxs, da = run(ldc, w)
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, 1, w.T - 1], rng.integers(0, w.T, 509)]))
    sw = dict(xs=[x[rows] for x in w.xs], a=w.a[rows], dys=[d[rows] for d in w.dys])
    ry = mo.forward(sw["xs"], sw["a"])
    rdx, rda = mo.backward(sw["xs"], sw["a"], sw["dys"])
    for k in range(w.W):
        check(f"y{k}", ys[k][rows], ry[k])
    for j in range(w.J):
        check(f"dx{j}", dxs[j][rows], rdx[j])
    check("da", da[rows], rda)


def test_deterministic(ldc):
    w = wl.make_mudd_workload(300, 768, 4, 13, seed=12)
    first = run(ldc, w)
    second = run(ldc, w)
    for u, v in zip([*first[0], *first[1], first[2]], [*second[0], *second[1], second[2]]):
        assert np.array_equal(u, v)


def test_one_hot_weights_copy_streams(ldc):
    """Selection by one-hot weights returns the selected stream exactly."""
    import torch
    from dynamic_head_composition_amd import mudd
    w = wl.make_mudd_workload(129, 768, 4, 6, seed=13)
    rng = np.random.default_rng(1)
    sel = rng.integers(0, w.J, size=(w.T, w.W))
    w.a[:] = 0.0
    for k in range(w.W):
        w.a[np.arange(w.T), k, sel[:, k]] = 1.0
    xs, a, _ = w.torch_inputs("cuda")
    ys = mudd.fwd(xs, a)
    torch.cuda.synchronize()
    for k in range(w.W):
        want = np.stack([w.xs[sel[t, k]][t] for t in range(w.T)])
        assert np.array_equal(ys[k].cpu().numpy(), want)


def test_binding_rejects_bad_shapes(ldc):
    import torch
    from dynamic_head_composition_amd import mudd
    x = torch.zeros((4, 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        mudd.fwd([x], torch.zeros((4, 1, 2), device="cuda"))
    with pytest.raises(ValueError):
        mudd.bwd([x], torch.zeros((4, 2, 1), device="cuda"), [x])


def test_autograd_matches_oracle(ldc):
    """mudd_mix through torch autograd: gradients of sum_w <dY_w, Y_w> with
    respect to the streams and the weights equal the oracle's backward."""
    import torch
    from dynamic_head_composition_amd import mudd
    w = wl.make_mudd_workload(77, 256, 2, 3, dtype="f32", seed=14)
    xs, a, dys = w.torch_inputs("cuda")
    xs = [x.requires_grad_() for x in xs]
    a.requires_grad_()
    ys = mudd.mudd_mix(xs, a)
    loss = sum((y * d).sum() for y, d in zip(ys, dys))
    loss.backward()
    rdx, rda = mo.backward(w.xs, w.a, w.dys)
    ry = mo.forward(w.xs, w.a)
    for k in range(w.W):
        check(f"y{k}", ys[k].detach().cpu().numpy(), ry[k])
    for j in range(w.J):
        check(f"dx{j}", xs[j].grad.cpu().numpy(), rdx[j])
    check("da", a.grad.cpu().numpy(), rda)
