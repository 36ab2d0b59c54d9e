"""GPU parity of the fused block (the Lightweight DC layer fused with the main
attention, forward) through the C ABI against the fp64 oracle
(oracle/fused_oracle.py): small and ragged streams element by element, the
full-size stream on sampled rows, the main attention alone, and determinism."""
import numpy as np
import pytest

from dynamic_head_composition_amd import workloads as wl
from oracle import fused_oracle as fo
from tests.helpers import assert_close, to_np

pytestmark = pytest.mark.gpu

REPEATED = np.array([0] * 100 + [1] * 50 + [0] * 200 + [2] * 106, dtype=np.int32)  # id 0 twice
# run boundaries on and beside the run-start pass's 1024-token block edges
EDGES = np.repeat(np.arange(7, dtype=np.int32), [1023, 1, 1025, 2047, 1, 3000, 130])

SMALL = [  # (T, H, d, window, docs, seed, c_kind)
    (1, 1, 64, 112, ("single",), 0, "normal0.5"),
    (17, 2, 64, 112, ("geometric", 6), 1, "normal0.5"),
    (300, 2, 128, 112, ("single",), 2, "normal0.5"),            # one run across two chunks
    (700, 3, 64, 113, ("uniform", 8, 256), 3, "onehot80"),
    (1000, 6, 128, 112, ("geometric", 300), 4, "normal0.5"),
    (1500, 4, 128, 37, ("single",), 5, "normal1neg"),          # up to 7 chunks before the window
    (333, 5, 64, 1, ("geometric", 100), 6, "normal0.5"),
    (2049, 6, 128, 112, ("geometric", 1024), 7, "normal0.5"),
    (456, 6, 64, 112, ("fixed", REPEATED), 8, "normal0.5"),      # a repeated id is a new document
    (129, 7, 128, 112, ("geometric", 40), 9, "normal0.5"),     # H = 7
    (len(EDGES), 2, 64, 112, ("fixed", EDGES), 10, "normal0.5"),
    # windows of 114-128 keys: the 10-block band, whose first block lies below the window stages
    (1100, 3, 128, 128, ("geometric", 300), 11, "normal0.5"),
    (700, 2, 64, 114, ("uniform", 8, 256), 12, "normal1neg"),
    (2049, 6, 128, 120, ("geometric", 1024), 13, "onehot80"),
    (150, 1, 64, 128, ("single",), 14, "normal0.5"),
]


@pytest.fixture(scope="module")
def fz(ldc):
    from dynamic_head_composition_amd import fused
    return fused


def inputs(w):
    x = w.torch_inputs("cuda", with_do=False)
    return x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"]


@pytest.mark.parametrize("T,H,d,window,docs,seed,ck", SMALL)
def test_parity_small(fz, T, H, d, window, docs, seed, ck):
    import torch
    w = wl.make_workload(T, H, d, window=window, docs=docs, seed=seed, c_kind=ck, with_do=False)
    print(f"case {w.name} window={window} recipe={w.recipe}", flush=True)
    q, k, v, c, g, doc = inputs(w)
    o = fz.fwd(q, k, v, c, g, doc, window=window, scale=w.scale)
    m = fz.main_fwd(q, k, v, doc, scale=w.scale)
    torch.cuda.synchronize()
    ref_m = fo.main_attention(w.q, w.k, w.v, w.doc, w.scale)
    ref_o = fo.forward(w.q, w.k, w.v, w.c, w.g, w.doc, window=window, scale=w.scale)
    assert_close("main", to_np(m), ref_m, "bf16")
    assert_close("o", to_np(o), ref_o, "bf16")


def test_matches_unfused_block(fz, ldc):
    """The fused output equals the main attention plus the Lightweight DC
    kernel's output (both GPU paths, fp32 rounding apart)."""
    import torch
    w = wl.make_workload(3000, 6, 128, docs=("geometric", 700), seed=30, with_do=False)
    q, k, v, c, g, doc = inputs(w)
    o = fz.fwd(q, k, v, c, g, doc, window=w.window, scale=w.scale)
    m = fz.main_fwd(q, k, v, doc, scale=w.scale)
    l_o = ldc.fwd(q, k, v, c, g, doc, window=w.window, scale=w.scale)
    torch.cuda.synchronize()
    got, want = to_np(o), to_np(m) + to_np(l_o)
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - want))) <= 2e-3


def test_deterministic(fz):
    import torch
    w = wl.make_workload(5000, 6, 128, docs=("geometric", 1024), seed=31, with_do=False)
    q, k, v, c, g, doc = inputs(w)
    a = fz.fwd(q, k, v, c, g, doc, window=w.window, scale=w.scale).clone()
    b = fz.fwd(q, k, v, c, g, doc, window=w.window, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def sampled_rows(T, rng, n=48):
    fixed = [0, 1, 63, 64, 127, 128, 191, 192, 4095, 4096, T // 2, T - 65, T - 64, T - 2, T - 1]
    return sorted(set(fixed) | set(int(x) for x in rng.integers(0, T, n - len(fixed))))


@pytest.mark.parametrize("cfg", [1, 4])
def test_full_size_sampled(fz, cfg):
    """The full-size stream in the benchmark's launch; rows the oracle computes
    one by one, each with its whole run and window."""
    import torch
    spec = dict(wl.CONFIGS[cfg])
    spec.pop("passes")
    w = wl.make_workload(**spec, with_do=False)
    print(f"case config {cfg} {w.name} recipe={w.recipe}", flush=True)
    q, k, v, c, g, doc = inputs(w)
    o = fz.fwd(q, k, v, c, g, doc, window=w.window, scale=w.scale)
    m = fz.main_fwd(q, k, v, doc, scale=w.scale)
    torch.cuda.synchronize()
    rows = sampled_rows(w.T, np.random.default_rng(100 + cfg))
    ref_o = fo.forward_rows(w.q, w.k, w.v, w.c, w.g, w.doc, rows, window=w.window, scale=w.scale)
    ref_m = fo.main_attention(w.q, w.k, w.v, w.doc, w.scale, queries=rows)
    assert_close("o rows", to_np(o)[rows], ref_o, "bf16")
    assert_close("main rows", to_np(m)[rows], ref_m, "bf16")
    assert np.all(np.isfinite(to_np(o)))


def test_long_document(fz):
    """One 12,288-token document: every tile walks the run from token 0."""
    import torch
    w = wl.make_workload(12288, 2, 64, docs=("single",), seed=32, with_do=False)
    q, k, v, c, g, doc = inputs(w)
    o = fz.fwd(q, k, v, c, g, doc, window=w.window, scale=w.scale)
    torch.cuda.synchronize()
    rows = sampled_rows(w.T, np.random.default_rng(7), n=24)
    ref = fo.forward_rows(w.q, w.k, w.v, w.c, w.g, w.doc, rows, window=w.window, scale=w.scale)
    assert_close("o rows", to_np(o)[rows], ref, "bf16")


def test_empty(fz):
    import torch
    q = torch.zeros(0, 6, 128, dtype=torch.bfloat16, device="cuda")
    c = torch.zeros(0, 6, device="cuda")
    doc = torch.zeros(0, dtype=torch.int32, device="cuda")
    assert fz.fwd(q, q, q, c, c, doc).shape == (0, 6, 128)
    assert fz.main_fwd(q, q, q, doc).shape == (0, 6, 128)


@pytest.mark.parametrize("window", [112, 128])
def test_saved_state_matches_layer_forward(fz, ldc, window):
    """The fused call's workspace holds the Lightweight DC layer's saved state
    exactly as ldc_fwd writes it (the same score pass), so the backward can
    take it."""
    import torch
    w = wl.make_workload(777, 6, 128, window=window, docs=("geometric", 200), seed=33, with_do=False)
    q, k, v, c, g, doc = inputs(w)
    _, saved = fz.fwd(q, k, v, c, g, doc, window=w.window, scale=w.scale, save=True)
    _, ref = ldc.fwd(q, k, v, c, g, doc, window=w.window, scale=w.scale, save=True)
    torch.cuda.synchronize()
    n = ldc.saved_bytes(ldc.LDC_BF16, w.T, w.H, w.d, w.window)
    assert torch.equal(saved[:n], ref.view(torch.uint8).reshape(-1)[:n])


def test_run_start_lookback(fz):
    """A run longer than 256 run-start blocks (262,144 tokens): the look-back
    over the block summaries takes a second round."""
    import torch
    T = 270000
    docs = np.zeros(T, dtype=np.int32)
    docs[5:] = 1
    w = wl.make_workload(T, 1, 64, docs=("fixed", docs), seed=34, with_do=False)
    q, k, v, c, g, doc = inputs(w)
    m = fz.main_fwd(q, k, v, doc, scale=w.scale)
    torch.cuda.synchronize()
    rows = [0, 4, 5, 6, 1023, 262143, 262144, 262150, T - 1]
    ref = fo.main_attention(w.q, w.k, w.v, w.doc, w.scale, queries=rows)
    assert_close("main rows", to_np(m)[rows], ref, "bf16")
