"""GPU parity of the C/G generator kernels (through the C ABI) against the
fp64 oracle (oracle/cg_oracle.py)."""
import numpy as np
import pytest

from dynamic_head_composition_amd import workloads as wl
from oracle import cg_oracle as cgo
from tests.helpers import assert_close, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cg(ldc):
    from dynamic_head_composition_amd import cg
    return cg


CASES = [  # (T, dm, H, dtype, seed)
    (1, 64, 1, "f32", 0),
    (17, 128, 3, "f32", 1),
    (300, 768, 6, "f32", 2),
    (1000, 768, 6, "bf16", 3),
    (257, 1024, 8, "bf16", 4),
    (4097, 768, 6, "bf16", 5),
    (33, 64, 2, "bf16", 6),
    # the forward's unrolled paths (dm = 256, 512 per 8-step batch of bf16,
    # 128 of fp32) with whole 64-token waves and a ragged last one
    (640, 256, 4, "bf16", 8),
    (333, 512, 7, "bf16", 9),
    (300, 256, 5, "f32", 10),
    (129, 384, 2, "f32", 11),
    (200, 512, 8, "f32", 12),
]


@pytest.mark.parametrize("T,dm,H,dtype,seed", CASES)
def test_parity(cg, T, dm, H, dtype, seed):
    import torch
    w = wl.make_cg_workload(T, dm, H, dtype=dtype, seed=seed)
    print(f"case {w.name}", flush=True)
    x = w.torch_inputs("cuda")
    c, g = cg.fwd(x["x"], x["wc"], x["wg"])
    dx, dwc, dwg = cg.bwd(x["x"], x["wc"], x["wg"], x["dc"], x["dg"])
    torch.cuda.synchronize()
    rc, rg = cgo.forward(w.x, w.wc, w.wg)
    rdx, rdwc, rdwg = cgo.backward(w.x, w.wc, w.wg, w.dc, w.dg)
    for name, got, ref in (("c", c, rc), ("g", g, rg), ("dx", dx, rdx), ("dwc", dwc, rdwc), ("dwg", dwg, rdwg)):
        assert_close(name, to_np(got), ref, dtype)


def test_full_size_and_determinism(cg):
    """The 65,536-token GPT-2 hidden state: whole tensors against the oracle,
    and bitwise-equal repeats."""
    import torch
    w = wl.make_cg_workload(**wl.CG_BENCH)
    x = w.torch_inputs("cuda")
    r1 = cg.fwd(x["x"], x["wc"], x["wg"]) + cg.bwd(x["x"], x["wc"], x["wg"], x["dc"], x["dg"])
    r2 = cg.fwd(x["x"], x["wc"], x["wg"]) + cg.bwd(x["x"], x["wc"], x["wg"], x["dc"], x["dg"])
    torch.cuda.synchronize()
    for a_, b_ in zip(r1, r2):
        assert torch.equal(a_, b_)
    refs = cgo.forward(w.x, w.wc, w.wg) + cgo.backward(w.x, w.wc, w.wg, w.dc, w.dg)
    for name, got, ref in zip(("c", "g", "dx", "dwc", "dwg"), r1, refs):
        assert_close(name, to_np(got), ref, "bf16")


def test_empty_stream_zeroes_weight_gradients(cg):
    import torch
    w = wl.make_cg_workload(8, 128, 4, dtype="bf16", seed=7)
    x = w.torch_inputs("cuda")
    empty = x["x"][:0]
    dwc = torch.full((128, 4), float("nan"), device="cuda")
    dwg = torch.full((128, 4), float("nan"), device="cuda")
    cg.bwd(empty, x["wc"], x["wg"], x["dc"][:0], x["dg"][:0], out=(torch.empty((0, 128), device="cuda"), dwc, dwg),
           workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(dwc == 0) and torch.all(dwg == 0)
