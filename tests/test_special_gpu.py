"""Properties the layer's definition fixes, checked on the HIP path directly
(GPU), beside the parity tests: invariance of the keys under a common shift,
equivariance under a permutation of whole documents, exact linearity of O in
C and G, and run-to-run determinism."""
import numpy as np
import pytest

from dynamic_head_composition_amd import workloads as wl
from tests.helpers import assert_close, run_gpu, to_np

pytestmark = pytest.mark.gpu

KEYS = ("o", "dq", "dk", "dv", "dc", "dg")


def test_key_shift_invariance(ldc):
    """Adding one vector u to every key of a head adds <Q[t], u> to a whole
    score row, which the softmax removes, so O, dV, dC, dG and dK (which depend
    on the keys only through P) are unchanged, and dQ gains sigma (sum_s dS) u
    = 0.  fp32 storage, so the shifted keys are exact up to fp32 rounding."""
    w = wl.make_workload(700, 3, 64, dtype="f32", seed=41, docs=("geometric", 200))
    base, _ = run_gpu(ldc, w)
    u = np.random.default_rng(1).standard_normal((1, w.H, w.d)).astype(np.float32)
    shifted = wl.Workload(**{**w.__dict__, "k": (w.k + u).astype(np.float32)})
    res, _ = run_gpu(ldc, shifted)
    for key in KEYS:
        assert_close(f"{key} shifted", to_np(res[key]), to_np(base[key]).astype(np.float64), "f32")


def test_document_permutation_equivariance(ldc):
    """Reordering whole documents reorders every per-token result the same way."""
    w = wl.make_workload(900, 2, 128, dtype="f32", seed=42, docs=("uniform", 20, 140))
    base, _ = run_gpu(ldc, w)
    bounds = np.flatnonzero(np.r_[True, w.doc[1:] != w.doc[:-1], True])
    docs = [np.arange(bounds[i], bounds[i + 1]) for i in range(len(bounds) - 1)]
    order = np.random.default_rng(3).permutation(len(docs))
    perm = np.concatenate([docs[i] for i in order])  # new token n is old token perm[n]
    fields = {f: getattr(w, f)[perm] for f in ("q", "k", "v", "c", "g", "do")}
    doc = np.concatenate([np.full(len(docs[i]), j, np.int32) for j, i in enumerate(order)])
    pw = wl.Workload(**{**w.__dict__, **fields, "doc": doc})
    res, _ = run_gpu(ldc, pw)
    for key in KEYS:
        assert_close(f"{key} permuted", to_np(res[key]),
                     to_np(base[key])[perm].astype(np.float64), "f32")


def test_linearity_in_c_and_g(ldc):
    """O is linear in G and in C: doubling either doubles O exactly (scaling by
    two is exact in every step, the bf16 hi/lo split included), and the layer
    is additive in C up to rounding."""
    import torch
    w = wl.make_workload(500, 6, 128, dtype="bf16", seed=43, docs=("geometric", 150))
    x = w.torch_inputs("cuda")

    def fwd(c, g):
        o = ldc.fwd(x["q"], x["k"], x["v"], c, g, x["doc"], window=w.window, scale=w.scale)
        torch.cuda.synchronize()
        return o

    o = fwd(x["c"], x["g"])
    assert torch.equal(fwd(x["c"], 2 * x["g"]), 2 * o)
    assert torch.equal(fwd(2 * x["c"], x["g"]), 2 * o)
    c1 = torch.randn(x["c"].shape, generator=torch.Generator(device="cuda").manual_seed(5), device="cuda")
    c2 = x["c"] - c1
    o12 = fwd(c1, x["g"]) + fwd(c2, x["g"])
    assert_close("O(C1) + O(C2) vs O(C1 + C2)", o12.cpu().numpy(),
                 o.cpu().numpy().astype(np.float64), "bf16")


def test_forward_bitwise_over_ten_runs(ldc):
    import torch
    w = wl.make_workload(2000, 6, 128, dtype="bf16", seed=44)
    x = w.torch_inputs("cuda")
    first, saved = ldc.fwd(x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"], window=w.window,
                           scale=w.scale, save=True)
    grads = ldc.bwd(x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"], saved, x["do"],
                    window=w.window, scale=w.scale)
    for _ in range(9):
        o, s2 = ldc.fwd(x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"], window=w.window,
                        scale=w.scale, save=True)
        assert torch.equal(o, first) and torch.equal(s2, saved)
    for _ in range(2):
        again = ldc.bwd(x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"], saved, x["do"],
                        window=w.window, scale=w.scale)
        for a, b in zip(again, grads):
            assert torch.equal(a, b)
