"""GPU parity of the DCMHA kernels (through the C ABI) against the fp64 oracle
(oracle/dcmha_oracle.py), the reduction to the Lightweight DC kernels, and
the backward's structural properties."""
import numpy as np
import pytest

from dynamic_head_composition_amd import workloads as wl
from oracle import dcmha_oracle as dco
from tests.helpers import assert_close, to_np

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dcs", "dcw")


@pytest.fixture(scope="module")
def dc(ldc):
    from dynamic_head_composition_amd import dcmha
    return dcmha


def run(dc, w, x=None, saved_state=True):
    import torch
    x = x or w.torch_inputs("cuda")
    args = (x["q"], x["k"], x["v"], x["cs"], x["cw"], x["doc"])
    o, saved = dc.fwd(*args, window=w.window, scale=w.scale, save=True)
    gr = dc.bwd(*args, saved if saved_state else None, x["do"], window=w.window, scale=w.scale)
    torch.cuda.synchronize()
    return dict(o=o, **dict(zip(GRADS, gr))), x


def oracle(w):
    o = dco.forward(w.q, w.k, w.v, w.cs, w.cw, w.doc, window=w.window, scale=w.scale)
    gr = dco.backward(w.q, w.k, w.v, w.cs, w.cw, w.doc, w.do, window=w.window, scale=w.scale)
    return dict(o=o, **dict(zip(GRADS, gr)))


SMALL = [  # (T, H, d, dtype, window, docs, seed, cs_kind, cw_kind)
    (1, 1, 64, "f32", 112, ("single",), 0, "eye+normal0.3", "eye+normal0.3"),
    (17, 2, 64, "f32", 112, ("geometric", 6), 1, "eye+normal0.3", "eye+normal0.3"),
    (300, 2, 64, "f32", 112, ("geometric", 90), 2, "eye+normal0.3", "eye+normal0.3"),
    (257, 3, 64, "f32", 113, ("uniform", 8, 64), 3, "eye+normal0.3", "eye+normal0.3"),
    (200, 6, 64, "f32", 5, ("geometric", 40), 4, "eye+normal0.3", "eye+normal0.3"),
    (150, 5, 64, "f32", 1, ("geometric", 30), 5, "eye+normal0.3", "eye+normal0.3"),
    (1000, 6, 128, "bf16", 112, ("geometric", 300), 6, "eye+normal0.3", "eye+normal0.3"),
    (700, 6, 64, "bf16", 112, ("uniform", 8, 256), 7, "eye+normal0.3", "eye+normal0.3"),
    (333, 4, 128, "bf16", 37, ("geometric", 100), 8, "eye+normal0.3", "eye+normal0.3"),
    (129, 2, 64, "bf16", 112, ("single",), 9, "eye+normal0.3", "eye+normal0.3"),
    (150, 1, 128, "bf16", 112, ("geometric", 50), 10, "eye+normal0.3", "eye+normal0.3"),
    (265, 3, 128, "bf16", 113, ("geometric", 60), 11, "perm", "perm"),
    (400, 6, 128, "bf16", 112, ("geometric", 120), 12, "eye", "eye"),
]


@pytest.mark.parametrize("T,H,d,dtype,window,docs,seed,csk,cwk", SMALL)
def test_parity_small(dc, T, H, d, dtype, window, docs, seed, csk, cwk):
    w = wl.make_dcmha_workload(T, H, d, dtype=dtype, window=window, docs=docs, seed=seed,
                               cs_kind=csk, cw_kind=cwk)
    print(f"case {w.name} window={window} recipe={w.recipe}", flush=True)
    res, _ = run(dc, w)
    ref = oracle(w)
    for key in ("o",) + GRADS:
        assert_close(key, to_np(res[key]), ref[key], dtype)


def test_parity_many_tiles(dc):
    """4,096 tokens: 64 query tiles and 32 key tiles, several per XCD."""
    w = wl.make_dcmha_workload(4096, 6, 128, dtype="bf16", seed=20)
    print(f"case {w.name} recipe={w.recipe}", flush=True)
    res, _ = run(dc, w)
    ref = oracle(w)
    for key in ("o",) + GRADS:
        assert_close(key, to_np(res[key]), ref[key], "bf16")


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_reduces_to_lightweight_dc_kernels(ldc, dc, dtype, d):
    """CS = I, CW[t,h,:] = G[t,h] C[t,:]: the DCMHA kernels give what the
    Lightweight DC kernels give; dC, dG follow from dCW by the chain rule."""
    import dataclasses
    import torch
    T, H = 900, 5
    lw = wl.make_workload(T, H, d, dtype=dtype, seed=21, docs=("geometric", 200))
    w = wl.make_dcmha_workload(T, H, d, dtype=dtype, seed=21, cs_kind="eye", cw_kind="eye")
    w = dataclasses.replace(w, q=lw.q, k=lw.k, v=lw.v, do=lw.do, doc=lw.doc,
                            cw=(lw.g[:, :, None] * lw.c[:, None, :]).astype(np.float32))
    res, _ = run(dc, w)
    lx = lw.torch_inputs("cuda")
    largs = (lx["q"], lx["k"], lx["v"], lx["c"], lx["g"], lx["doc"])
    o, saved = ldc.fwd(*largs, window=w.window, scale=w.scale, save=True)
    lg = ldc.bwd(*largs, saved, lx["do"], window=w.window, scale=w.scale)
    torch.cuda.synchronize()
    ref = lambda t: to_np(t).astype(np.float64)
    assert_close("o", to_np(res["o"]), ref(o), dtype)
    for name, a_, b_ in zip(("dq", "dk", "dv"), (res["dq"], res["dk"], res["dv"]), lg[:3]):
        assert_close(name, to_np(a_), ref(b_), dtype)
    dcw = ref(res["dcw"])
    assert_close("dc", np.einsum("th,thg->tg", lw.g.astype(np.float64), dcw), ref(lg[3]), dtype)
    assert_close("dg", np.einsum("tg,thg->th", lw.c.astype(np.float64), dcw), ref(lg[4]), dtype)


def test_backward_without_saved_state_is_bitwise_equal(dc):
    import torch
    w = wl.make_dcmha_workload(2000, 6, 128, dtype="bf16", seed=22)
    a, x = run(dc, w, saved_state=True)
    b, _ = run(dc, w, x, saved_state=False)
    for key in GRADS:
        assert torch.equal(a[key], b[key]), key


def test_parts_equal_whole_backward(dc):
    import torch
    w = wl.make_dcmha_workload(1500, 6, 64, dtype="bf16", seed=23)
    x = w.torch_inputs("cuda")
    args = (x["q"], x["k"], x["v"], x["cs"], x["cw"], x["doc"])
    _, saved = dc.fwd(*args, window=w.window, scale=w.scale, save=True)
    whole = dc.bwd(*args, saved, x["do"], window=w.window, scale=w.scale)
    ws = torch.empty(dc.workspace_bytes(0, w.T, w.H, w.d, w.window), dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    outs = tuple(torch.full(s, float("nan"), **f32) for s in ((w.T, w.H, w.d),) * 3 + ((w.T, w.H, w.H),) * 2)
    dc.bwd(*args, saved, x["do"], window=w.window, scale=w.scale, out=outs, workspace=ws, part="q")
    dc.bwd(*args, saved, x["do"], window=w.window, scale=w.scale, out=outs, workspace=ws, part="kv")
    torch.cuda.synchronize()
    for name, a_, b_ in zip(GRADS, whole, outs):
        assert torch.equal(a_, b_), name


def test_deterministic(dc):
    import torch
    w = wl.make_dcmha_workload(3000, 6, 128, dtype="bf16", seed=24)
    a, x = run(dc, w)
    b, _ = run(dc, w, x)
    for key in ("o",) + GRADS:
        assert torch.equal(a[key], b[key]), key


def test_autograd_function_bf16(dc):
    import torch
    w = wl.make_dcmha_workload(600, 6, 128, dtype="bf16", seed=25)
    x = w.torch_inputs("cuda")
    q, k, v = (x[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    cs, cw = (x[n].clone().requires_grad_(True) for n in ("cs", "cw"))
    o = dc.dcmha_attention(q, k, v, cs, cw, x["doc"], window=w.window, scale=w.scale)
    assert o.dtype == torch.float32
    o.backward(x["do"].to(torch.float32))
    ref = oracle(w)
    assert_close("o", to_np(o), ref["o"], "bf16")
    for name, t in zip(GRADS, (q, k, v, cs, cw)):
        assert_close(name, to_np(t.grad), ref[name], "bf16")


def test_full_size_gpt2_shape(dc):
    """The benchmark workload (65,536 tokens, 6 x 128): whole-tensor identities
    and oracle values on three slices of 1,024 queries (with their halos)."""
    import torch
    cfg = dict(wl.DCMHA_BENCH)
    w = wl.make_dcmha_workload(**cfg)
    res, _ = run(dc, w)
    r = {k_: to_np(v_).astype(np.float64) for k_, v_ in res.items()}
    for key in r:
        assert np.all(np.isfinite(r[key])), key
    # <dV,V> = <dCW,CW> = <dO,O>;  <dCS,CS> = <dQ,Q> = <dK,K>
    ref = float(np.sum(w.do.astype(np.float64) * r["o"]))
    for x_, dx in ((w.v, r["dv"]), (w.cw, r["dcw"])):
        assert abs(float(np.sum(x_.astype(np.float64) * dx)) - ref) <= 2e-3 * abs(ref)
    sq = float(np.sum(w.q.astype(np.float64) * r["dq"]))
    for x_, dx in ((w.cs, r["dcs"]), (w.k, r["dk"])):
        assert abs(float(np.sum(x_.astype(np.float64) * dx)) - sq) <= 2e-3 * abs(sq)
    W = w.window
    for lo in (0, 31_000, w.T - 1024):
        hi = lo + 1024
        a0, a1 = max(0, lo - W + 1), min(w.T, hi + W - 1)
        sl = lambda x_: x_[a0:a1]
        o = dco.forward(sl(w.q), sl(w.k), sl(w.v), sl(w.cs), sl(w.cw), sl(w.doc), window=W, scale=w.scale)
        gr = dco.backward(sl(w.q), sl(w.k), sl(w.v), sl(w.cs), sl(w.cw), sl(w.doc), sl(w.do), window=W,
                          scale=w.scale)
        ref_ = dict(o=o, **dict(zip(GRADS, gr)))
        for key in ("o",) + GRADS:
            assert_close(f"{key}[{lo}:{hi}]", r[key][lo:hi], ref_[key][lo - a0:hi - a0], "bf16")
