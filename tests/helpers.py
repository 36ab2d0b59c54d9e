"""Shared helpers of the GPU parity tests: tolerances and runners."""
import numpy as np

# Tolerances: bf16 storage -> max abs <= 2e-2 and relative L2 <= 5e-3;
# fp32 storage -> relative L2 <= 1e-5 and max abs <= 1e-5 * max|ref|.
BF16_MAX_ABS, BF16_REL_L2 = 2e-2, 5e-3
F32_REL = 1e-5


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff)) / nref if nref > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_close(name, got, ref, dtype):
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    max_abs, rel = errors(got, ref)
    if dtype == "bf16":
        ok = max_abs <= BF16_MAX_ABS and rel <= BF16_REL_L2
        bound = f"max_abs<={BF16_MAX_ABS}, rel_l2<={BF16_REL_L2}"
    else:
        scale = float(np.max(np.abs(ref))) if ref.size else 0.0
        ok = rel <= F32_REL and max_abs <= F32_REL * max(scale, 1e-30)
        bound = f"rel_l2<={F32_REL}, max_abs<={F32_REL}*{scale:.3g}"
    msg = f"{name}: max_abs={max_abs:.3e} rel_l2={rel:.3e} ({bound})"
    print(msg, flush=True)
    assert ok, msg
    return max_abs, rel


def to_np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy()


def run_gpu(ldc, w, backward=True, window=None):
    """Forward (and backward) of workload w through the C ABI; numpy results."""
    import torch
    x = w.torch_inputs("cuda", with_do=backward)
    win = w.window if window is None else window
    o, saved = ldc.fwd(x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"], window=win, scale=w.scale,
                       save=True)
    res = {"o": o}
    if backward:
        dq, dk, dv, dc, dg = ldc.bwd(x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"], saved, x["do"],
                                     window=win, scale=w.scale)
        res.update(dq=dq, dk=dk, dv=dv, dc=dc, dg=dg)
    torch.cuda.synchronize()
    return res, x
