"""GPU parity at the five reference workloads' full sizes, in the launch
configuration the benchmark times (the same entry points on the whole stream).

Forward: the whole output tensor of every workload.  Backward: seeded
4,096-token slices (the oracle runs each slice with its window halo, so the
compared rows are exact) plus the stream's first and last rows, and
full-tensor invariants of the gradients."""
import numpy as np
import pytest

from dynamic_head_composition_amd import workloads as wl
from oracle import ldc_oracle as orc
from tests.helpers import BF16_REL_L2, assert_close, to_np

pytestmark = pytest.mark.gpu

SLICE = 4096
_cache = {}


def workload(i):
    if i not in _cache:
        _cache.clear()
        print(f"generating workload {i}", flush=True)
        _cache[i] = wl.config_workload(i)
    return _cache[i]


def run_full(ldc, w, backward):
    import torch
    x = w.torch_inputs("cuda", with_do=backward)
    o, saved = ldc.fwd(x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"], window=w.window,
                       scale=w.scale, save=True)
    res = {"o": o}
    if backward:
        res.update(zip(("dq", "dk", "dv", "dc", "dg"),
                       ldc.bwd(x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"], saved, x["do"],
                               window=w.window, scale=w.scale)))
    torch.cuda.synchronize()
    for key, val in res.items():
        assert bool(torch.isfinite(val).all()), key
    return res, x


def slice_starts(w, i):
    rng = np.random.default_rng(100 + i)
    return [0, int(rng.integers(SLICE, w.T - 2 * SLICE)), w.T - SLICE]


def check_bwd_slices(w, res, starts):
    for a in starts:
        ref = orc.backward_slice(w.q, w.k, w.v, w.c, w.g, w.doc, w.do, a, a + SLICE,
                                 window=w.window, scale=w.scale)
        for key, r in zip(("dq", "dk", "dv", "dc", "dg"), ref):
            assert_close(f"{key}[{a}:{a + SLICE}]", to_np(res[key][a:a + SLICE]), r, w.dtype)


def check_invariants(w, res, x):
    """Whole-stream properties of the gradients (float64 on the GPU):
    per token  sum_h C dC = sum_h G dG;  per (t,h)  G dG = <dO, O>;
    per document and head  sum dK = 0  and  sum dV = sum_t G (sum_h' C) dO."""
    import torch
    f64 = lambda t: t.to(torch.float64)
    c, g, do = f64(x["c"]), f64(x["g"]), f64(x["do"])
    dq, dk, dv, dc, dg, o = (f64(res[k]) for k in ("dq", "dk", "dv", "dc", "dg", "o"))

    def rel(a, b, scale=None):
        return float(torch.linalg.norm(a - b) / torch.linalg.norm(b if scale is None else scale))

    r1 = rel((c * dc).sum(1), (g * dg).sum(1))
    r2 = rel(g * dg, (do * o).sum(-1))
    doc = x["doc"].long()
    ndoc = int(doc.max()) + 1
    sdk = torch.zeros((ndoc,) + dk.shape[1:], dtype=torch.float64, device=dk.device).index_add_(0, doc, dk)
    sdv = torch.zeros_like(sdk).index_add_(0, doc, dv)
    ref_dv = torch.zeros_like(sdk).index_add_(0, doc, g[:, :, None] * c.sum(1)[:, None, None] * do)
    r3 = float(torch.linalg.norm(sdk) / torch.linalg.norm(dk))
    r4 = rel(sdv, ref_dv)
    print(f"invariants: C.dC=G.dG {r1:.2e}  G.dG=<dO,O> {r2:.2e}  sum dK {r3:.2e}  sum dV {r4:.2e}", flush=True)
    for name, r in (("C.dC=G.dG", r1), ("G.dG=<dO,O>", r2), ("doc sum dK=0", r3), ("doc sum dV", r4)):
        assert r <= BF16_REL_L2, (name, r)


def test_cfg1_gpt2_small_forward_full_tensor(ldc):
    w = workload(1)
    res, _ = run_full(ldc, w, backward=False)
    ref = orc.forward(w.q, w.k, w.v, w.c, w.g, w.doc, window=w.window, scale=w.scale)
    assert_close("o (all 65536 tokens)", to_np(res["o"]), ref, w.dtype)


@pytest.mark.parametrize("i", [2, 3, 4])
def test_fwd_bwd_full_size(ldc, i):
    w = workload(i)
    print(f"workload {w.name}: {w.recipe}", flush=True)
    res, x = run_full(ldc, w, backward=True)
    ref = orc.forward(w.q, w.k, w.v, w.c, w.g, w.doc, window=w.window, scale=w.scale)
    assert_close(f"o (all {w.T} tokens)", to_np(res["o"]), ref, w.dtype)
    del ref
    starts = slice_starts(w, i)
    check_bwd_slices(w, res, starts)
    check_invariants(w, res, x)
