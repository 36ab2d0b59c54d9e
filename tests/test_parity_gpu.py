"""GPU parity of the HIP path (through the C ABI) against the fp64 CPU oracle
on small and ragged inputs, special cases and edge cases."""
import math

import numpy as np
import pytest

from dynamic_head_composition_amd import workloads as wl
from oracle import ldc_oracle as orc
from tests.helpers import assert_close, run_gpu, to_np

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dc", "dg")


def oracle_all(w, window=None):
    win = w.window if window is None else window
    o = orc.forward(w.q, w.k, w.v, w.c, w.g, w.doc, window=win, scale=w.scale)
    gr = orc.backward(w.q, w.k, w.v, w.c, w.g, w.doc, w.do, window=win, scale=w.scale)
    return dict(o=o, **dict(zip(GRADS, gr)))


def check_all(ldc, w, window=None, backward=True):
    print(f"case {w.name} window={window or w.window} recipe={w.recipe}", flush=True)
    res, _ = run_gpu(ldc, w, backward=backward, window=window)
    ref = oracle_all(w, window)
    for key in ("o",) + (GRADS if backward else ()):
        assert_close(key, to_np(res[key]), ref[key], w.dtype)


SMALL = [  # (T, H, d, dtype, window, docs, seed)
    (1, 1, 16, "f32", 112, ("single",), 0),
    (17, 2, 16, "f32", 112, ("geometric", 6), 1),
    (300, 2, 16, "f32", 112, ("geometric", 90), 2),
    (300, 3, 64, "f32", 5, ("geometric", 40), 3),
    (257, 2, 128, "f32", 113, ("uniform", 8, 64), 4),
    (200, 1, 64, "f32", 1, ("geometric", 30), 5),
    (1000, 6, 128, "bf16", 112, ("geometric", 300), 6),
    (1000, 12, 64, "bf16", 112, ("uniform", 8, 256), 7),
    (333, 6, 128, "bf16", 37, ("geometric", 100), 8),
    (129, 2, 64, "bf16", 112, ("single",), 9),
    # odd head counts (a padding stage closes each phase), the widest window
    (500, 3, 128, "bf16", 113, ("geometric", 150), 20),
    (400, 5, 64, "bf16", 100, ("uniform", 8, 64), 21),
    # a whole number of 128-token tiles; several tiles per XCD
    (256, 6, 128, "bf16", 112, ("single",), 22),
    (4096, 6, 128, "bf16", 112, ("geometric", 1024), 23),
    # the last wave holds 9 and 8 rows: the whole-line row stores have one
    # and zero active lanes in their second half
    (265, 2, 128, "bf16", 112, ("geometric", 60), 24),
    (136, 4, 64, "bf16", 64, ("uniform", 8, 40), 25),
    # one head on the bf16 paths (a single real stage and a padding stage per
    # phase), and sixteen heads of 64 (GPT-2 medium's attention shape)
    (150, 1, 128, "bf16", 112, ("geometric", 50), 26),
    (97, 1, 64, "bf16", 20, ("uniform", 8, 30), 27),
    (300, 16, 64, "bf16", 112, ("geometric", 80), 28),
    # bf16 rows of 16 (the K = 16 MFMA paths): the tiny configuration's shape
    # in bf16, ragged streams, several tiles, windows 1 and 113
    (256, 2, 16, "bf16", 112, ("fixed", np.array([0] * 100 + [1] * 156, dtype=np.int32)), 29),
    (17, 3, 16, "bf16", 112, ("geometric", 6), 30),
    (1000, 6, 16, "bf16", 113, ("geometric", 200), 31),
    (333, 4, 16, "bf16", 1, ("uniform", 8, 64), 32),
    (4096, 12, 16, "bf16", 112, ("geometric", 1024), 33),
]


@pytest.mark.parametrize("T,H,d,dtype,window,docs,seed", SMALL)
def test_small_fwd_bwd(ldc, T, H, d, dtype, window, docs, seed):
    w = wl.make_workload(T, H, d, dtype=dtype, window=window, docs=docs, seed=seed)
    check_all(ldc, w)


def test_cfg0_tiny_forward(ldc):
    w = wl.config_workload(0)
    check_all(ldc, w, backward=False)


def test_cfg0_tiny_backward(ldc):
    # the tiny configuration is quoted forward-only; its backward is checked too
    check_all(ldc, wl.config_workload(0))


def test_every_token_its_own_document(ldc):
    T = 300
    w = wl.make_workload(T, 2, 64, dtype="f32", docs=("fixed", np.arange(T, dtype=np.int32)), seed=11)
    check_all(ldc, w)
    res, _ = run_gpu(ldc, w)
    # closed form: single-key windows
    np.testing.assert_allclose(to_np(res["o"]), w.g[:, :, None] * w.c.sum(1)[:, None, None] * w.v,
                               rtol=1e-5, atol=1e-5)
    # dQ comes from the query-side pass, which sees P = 1 exactly
    assert np.all(to_np(res["dq"]) == 0)
    assert np.max(np.abs(to_np(res["dk"]))) <= 1e-5


def test_arbitrary_doc_labels(ldc):
    """doc_ids are compared for equality only: interleaved labels make every
    other token a document of its own kind."""
    T = 400
    doc = (np.arange(T) % 3 == 0).astype(np.int32) * 7 - 2
    w = wl.make_workload(T, 2, 64, dtype="f32", docs=("fixed", doc), seed=12)
    check_all(ldc, w)


def test_window_one_closed_form_bf16(ldc):
    w = wl.make_workload(500, 6, 128, dtype="bf16", seed=13, docs=("geometric", 50))
    res, _ = run_gpu(ldc, w, window=1)
    ref = w.g[:, :, None] * w.c.sum(1)[:, None, None] * w.v
    assert_close("o", to_np(res["o"]), ref, "bf16")
    assert np.all(to_np(res["dq"]) == 0)
    assert np.max(np.abs(to_np(res["dk"]))) <= 1e-4


def test_onehot_composition(ldc):
    """C = one-hot(h*) and G = 1: head h*'s map drives every head."""
    w = wl.make_workload(700, 6, 128, dtype="f32", seed=14, docs=("geometric", 200), g_kind="one")
    w.c[:] = 0.0
    w.c[:, 4] = 1.0
    check_all(ldc, w)


def test_constant_values(ldc):
    """G = 1, rows of C summing to 1, V constant per head: O = V."""
    w = wl.make_workload(600, 6, 128, dtype="bf16", seed=15, g_kind="one")
    w.c[:] = w.c - w.c.mean(1, keepdims=True) + 1.0 / 6
    vh = wl.round_bf16(np.random.default_rng(16).standard_normal((6, 128)).astype(np.float32))
    w.v[:] = vh[None]
    res, _ = run_gpu(ldc, w, backward=False)
    assert_close("o", to_np(res["o"]), np.broadcast_to(vh[None], w.v.shape), "bf16")


def test_document_starts(ldc):
    w = wl.make_workload(2000, 6, 128, dtype="bf16", seed=17, docs=("geometric", 64))
    res, _ = run_gpu(ldc, w)
    starts = np.nonzero(np.r_[True, w.doc[1:] != w.doc[:-1]])[0]
    o = to_np(res["o"])[starts]
    ref = w.g[starts][:, :, None] * w.c[starts].sum(1)[:, None, None] * w.v[starts]
    assert_close("o@starts", o, ref, "bf16")
    assert np.all(to_np(res["dq"])[starts] == 0)


def test_hand_worked_example(ldc):
    """The hand-derived T=5 example (tests/golden), padded to head_dim 16 with zeros."""
    from tests.test_oracle_pins import load_golden
    gd, x, e = load_golden()
    T, H = gd["T"], gd["H"]
    pad = lambda a: np.concatenate([a, np.zeros((T, H, 15))], axis=2).astype(np.float32)
    w = wl.Workload(name="hand_T5", T=T, H=H, d=16, window=gd["window"], dtype="f32", scale=gd["scale"],
                    q=pad(x["q"]), k=pad(x["k"]), v=pad(x["v"]), c=x["c"].astype(np.float32),
                    g=x["g"].astype(np.float32), doc=x["doc"], do=pad(x["do"]))
    res, _ = run_gpu(ldc, w)
    for key in ("o", "dq", "dk", "dv"):
        got = to_np(res[key])
        assert_close(key, got[:, :, 0], e[key], "f32")
        assert np.all(got[:, :, 1:] == 0)
    for key in ("dc", "dg"):
        assert_close(key, to_np(res[key]), e[key], "f32")


def test_deterministic(ldc):
    import torch
    w = wl.make_workload(3000, 6, 128, dtype="bf16", seed=18)
    r1, _ = run_gpu(ldc, w)
    r2, _ = run_gpu(ldc, w)
    for key in r1:
        assert torch.equal(r1[key], r2[key]), key


def test_empty_stream(ldc):
    import torch
    z = torch.empty((0, 6, 128), dtype=torch.bfloat16, device="cuda")
    zc = torch.empty((0, 6), dtype=torch.float32, device="cuda")
    zd = torch.empty((0,), dtype=torch.int32, device="cuda")
    o, saved = ldc.fwd(z, z, z, zc, zc, zd, save=True)
    assert o.shape == (0, 6, 128)
    out = ldc.bwd(z, z, z, zc, zc, zd, saved, z)
    assert out[0].shape == (0, 6, 128)


def test_autograd_function(ldc):
    import torch
    w = wl.make_workload(256, 2, 64, dtype="f32", seed=19)
    x = w.torch_inputs("cuda")
    ts = {kk: x[kk].clone().requires_grad_(True) for kk in ("q", "k", "v", "c", "g")}
    o = ldc.ldc_attention(ts["q"], ts["k"], ts["v"], ts["c"], ts["g"], x["doc"], w.window, w.scale)
    o.backward(x["do"])
    gr = orc.backward(w.q, w.k, w.v, w.c, w.g, w.doc, w.do, window=w.window, scale=w.scale)
    for name, ref in zip(("q", "k", "v", "c", "g"), gr):
        assert_close("d" + name, to_np(ts[name].grad), ref, "f32")


def test_autograd_function_bf16(ldc):
    """ldc_attention on bf16 inputs: O comes back in float32 and meets the bf16
    bar; the gradients of the bf16 leaves are the kernels' float32 gradients
    rounded to bf16 by autograd (a leaf's gradient takes the leaf's dtype), and
    still meet the bf16 bar; C and G are float32 leaves."""
    import torch
    w = wl.make_workload(384, 6, 128, dtype="bf16", seed=31, docs=("geometric", 150))
    x = w.torch_inputs("cuda")
    ts = {kk: x[kk].clone().requires_grad_(True) for kk in ("q", "k", "v", "c", "g")}
    o = ldc.ldc_attention(ts["q"], ts["k"], ts["v"], ts["c"], ts["g"], x["doc"], w.window, w.scale)
    assert o.dtype == torch.float32
    o.backward(x["do"].float())
    ref_o = orc.forward(w.q, w.k, w.v, w.c, w.g, w.doc, window=w.window, scale=w.scale)
    assert_close("o", to_np(o), ref_o, "bf16")
    gr = orc.backward(w.q, w.k, w.v, w.c, w.g, w.doc, w.do, window=w.window, scale=w.scale)
    for name, ref in zip(("q", "k", "v", "c", "g"), gr):
        assert ts[name].grad.dtype == ts[name].dtype
        assert_close("d" + name, to_np(ts[name].grad), ref, "bf16")


def test_explicit_stream_argument(ldc):
    """stream= passed outside a stream context: the calls allocate their
    outputs, saved state and workspace on that stream and give the
    default-stream result bit for bit."""
    import torch
    w = wl.make_workload(600, 6, 128, dtype="bf16", seed=27)
    ref, _ = run_gpu(ldc, w)
    x = w.torch_inputs("cuda", with_do=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    args = (x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"])
    o, saved = ldc.fwd(*args, window=w.window, scale=w.scale, save=True, stream=s)
    grads = ldc.bwd(*args, saved, x["do"], window=w.window, scale=w.scale, stream=s)
    # more allocations on the current stream while s may still run
    junk = [torch.full((1 << 20,), 7.0, device="cuda") for _ in range(8)]
    s.synchronize()
    del junk
    assert torch.equal(o, ref["o"])
    for name, gr in zip(GRADS, grads):
        assert torch.equal(gr, ref[name]), name


def test_kv_part_needs_workspace(ldc):
    w = wl.make_workload(64, 2, 64, dtype="bf16", seed=28)
    x = w.torch_inputs("cuda", with_do=True)
    args = (x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"])
    _, saved = ldc.fwd(*args, save=True)
    with pytest.raises(ValueError):
        ldc.bwd(*args, saved, x["do"], part="kv")


@pytest.mark.parametrize("T,H,d,dtype,window", [(700, 6, 128, "bf16", 112), (300, 3, 64, "f32", 37),
                                                  (1000, 12, 64, "bf16", 112)])
def test_backward_without_saved_state(ldc, T, H, d, dtype, window):
    """ldc_bwd with saved = NULL recomputes the shared map and statistics
    (the forward's score phase) into its workspace: the gradients equal the
    call with the forward's saved state bit for bit, and the oracle's."""
    import torch
    w = wl.make_workload(T, H, d, dtype=dtype, window=window, seed=29, docs=("geometric", 150))
    x = w.torch_inputs("cuda", with_do=True)
    args = (x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"])
    _, saved = ldc.fwd(*args, window=w.window, scale=w.scale, save=True)
    with_state = ldc.bwd(*args, saved, x["do"], window=w.window, scale=w.scale)
    without = ldc.bwd(*args, None, x["do"], window=w.window, scale=w.scale)
    torch.cuda.synchronize()
    ref = orc.backward(w.q, w.k, w.v, w.c, w.g, w.doc, w.do, window=w.window, scale=w.scale)
    for name, a_, b_, r in zip(GRADS, with_state, without, ref):
        assert torch.equal(a_, b_), name
        assert_close(name, to_np(b_), r, w.dtype)


def test_split_backward_matches(ldc):
    """ldc_bwd_q then ldc_bwd_kv on one workspace gives exactly ldc_bwd."""
    import torch
    w = wl.make_workload(700, 6, 128, dtype="bf16", seed=24)
    x = w.torch_inputs("cuda", with_do=True)
    args = (x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"])
    _, saved = ldc.fwd(*args, window=w.window, scale=w.scale, save=True)
    full = ldc.bwd(*args, saved, x["do"], window=w.window, scale=w.scale)
    ws = torch.empty(ldc.workspace_bytes(ldc.LDC_BF16, 700, 6, 128, w.window), dtype=torch.uint8,
                     device="cuda")
    outs = tuple(torch.empty_like(t) for t in full)
    ldc.bwd(*args, saved, x["do"], window=w.window, scale=w.scale, out=outs, workspace=ws, part="q")
    ldc.bwd(*args, saved, x["do"], window=w.window, scale=w.scale, out=outs, workspace=ws, part="kv")
    torch.cuda.synchronize()
    for name, a_, b_ in zip(GRADS, full, outs):
        assert torch.equal(a_, b_), name


@pytest.mark.parametrize("T,H,d,dtype,seed", [(8192, 6, 128, "bf16", 51), (5000, 12, 64, "bf16", 52),
                                              (2000, 3, 64, "f32", 53), (700, 2, 128, "f32", 54)])
def test_backward_whole_tensor(ldc, T, H, d, dtype, seed):
    """Every gradient over the whole stream against the oracle, for streams of
    many tiles (64 of 128 tokens, 63 of 64 tokens at 12 x 64 and float32)."""
    w = wl.make_workload(T, H, d, dtype=dtype, seed=seed, docs=("geometric", 300))
    check_all(ldc, w)


def test_workspace_reuse(ldc):
    """Back-to-back calls on one workspace, with and without saved state,
    give identical results."""
    import torch
    w = wl.make_workload(3000, 6, 128, dtype="bf16", seed=55)
    x = w.torch_inputs("cuda", with_do=True)
    args = (x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"])
    _, saved = ldc.fwd(*args, window=w.window, scale=w.scale, save=True)
    ws = torch.empty(ldc.workspace_bytes(ldc.LDC_BF16, 3000, 6, 128, w.window), dtype=torch.uint8,
                     device="cuda")
    r1 = ldc.bwd(*args, saved, x["do"], window=w.window, scale=w.scale, workspace=ws)
    r2 = ldc.bwd(*args, saved, x["do"], window=w.window, scale=w.scale, workspace=ws)
    r3 = ldc.bwd(*args, None, x["do"], window=w.window, scale=w.scale, workspace=ws)
    torch.cuda.synchronize()
    for name, a_, b_, c_ in zip(GRADS, r1, r2, r3):
        assert torch.equal(a_, b_) and torch.equal(a_, c_), name


def test_custom_scale(ldc):
    """A softmax scale other than 1/sqrt(d) is honoured by both passes."""
    w = wl.make_workload(300, 2, 128, dtype="bf16", seed=25, scale=0.37)
    check_all(ldc, w)


def test_side_stream(ldc):
    """Work enqueued on a non-default stream gives the default-stream result."""
    import torch
    w = wl.make_workload(600, 6, 128, dtype="bf16", seed=26)
    ref, _ = run_gpu(ldc, w)
    x = w.torch_inputs("cuda", with_do=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o, saved = ldc.fwd(x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"], window=w.window,
                           scale=w.scale, save=True)
        grads = ldc.bwd(x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"], saved, x["do"],
                        window=w.window, scale=w.scale)
    s.synchronize()
    assert torch.equal(o, ref["o"])
    for name, gr in zip(GRADS, grads):
        assert torch.equal(gr, ref[name]), name


WIDE = [  # windows of 114..128 keys (10-block bands): (T, H, d, dtype, window, docs, seed)
    (1, 1, 16, "f32", 128, ("single",), 40),
    (300, 2, 16, "f32", 128, ("geometric", 90), 41),
    (257, 3, 64, "f32", 114, ("uniform", 8, 200), 42),
    (500, 6, 128, "bf16", 128, ("geometric", 300), 43),
    (1000, 12, 64, "bf16", 120, ("single",), 44),
    (129, 1, 128, "bf16", 127, ("single",), 45),
    (700, 5, 64, "bf16", 116, ("geometric", 150), 46),
    (600, 6, 16, "bf16", 128, ("geometric", 200), 49),
    (4096, 6, 128, "bf16", 128, ("geometric", 1024), 47),
]


@pytest.mark.parametrize("T,H,d,dtype,window,docs,seed", WIDE)
def test_wide_windows(ldc, T, H, d, dtype, window, docs, seed):
    w = wl.make_workload(T, H, d, dtype=dtype, window=window, docs=docs, seed=seed)
    check_all(ldc, w)


def test_wide_window_without_saved_state(ldc):
    """Window 128: the backward's own recomputation of the saved state gives
    bitwise the gradients of the saved one."""
    import torch
    w = wl.make_workload(2500, 6, 128, dtype="bf16", window=128, seed=48)
    x = w.torch_inputs("cuda", with_do=True)
    args = (x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"])
    _, saved = ldc.fwd(*args, window=128, scale=w.scale, save=True)
    a = ldc.bwd(*args, saved, x["do"], window=128, scale=w.scale)
    b = ldc.bwd(*args, None, x["do"], window=128, scale=w.scale)
    torch.cuda.synchronize()
    for name, a_, b_ in zip(GRADS, a, b):
        assert torch.equal(a_, b_), name
