"""ldc_bwd_noalloc (the backward entry point that allocates nothing and uses
the library's static per-GPU scratch as workspace) against ldc_bwd, through
the C ABI: bitwise-equal gradients on calls in a row, the later ones smaller,
with and without saved state."""
import pytest

from dynamic_head_composition_amd import workloads as wl

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dc", "dg")


def grads_like(torch, T, H, d):
    f32 = dict(dtype=torch.float32, device="cuda")
    return tuple(torch.full(s, float("nan"), **f32) for s in ((T, H, d),) * 3 + ((T, H),) * 2)


def case(ldc, T, H, d, dtype, seed, with_saved):
    import torch
    w = wl.make_workload(T, H, d, dtype=dtype, seed=seed, docs=("geometric", 300))
    x = w.torch_inputs("cuda", with_do=True)
    args = (x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"])
    saved = None
    if with_saved:
        _, saved = ldc.fwd(*args, window=w.window, scale=w.scale, save=True)
    return w, x, args, saved


@pytest.mark.parametrize("sizes", [
    # bf16 with saved state: the GPT-2 small layer's full stream, then a ragged smaller one
    [(65536, 6, 128, "bf16", 61, True), (1234, 6, 128, "bf16", 62, True)],
    # without saved state (the scratch also holds the recomputed state), f32 and bf16
    [(3000, 12, 64, "bf16", 63, False), (700, 2, 64, "f32", 64, False), (129, 3, 16, "f32", 65, True)],
])
def test_noalloc_matches_bwd(ldc, sizes):
    import torch
    print("noalloc cases", sizes, flush=True)
    assert ldc.noalloc_max_workspace() == 64 << 20
    cases = [case(ldc, *s) for s in sizes]
    outs = []
    for w, x, args, saved in cases:  # calls in a row on the shared scratch
        out = grads_like(torch, w.T, w.H, w.d)
        ldc.bwd_noalloc(*args, saved, x["do"], out, window=w.window, scale=w.scale)
        outs.append(out)
    torch.cuda.synchronize()
    for (w, x, args, saved), got in zip(cases, outs):
        ref = ldc.bwd(*args, saved, x["do"], window=w.window, scale=w.scale)
        torch.cuda.synchronize()
        for name, a_, b_ in zip(GRADS, got, ref):
            assert torch.equal(a_, b_), (w.name, name, float((a_ - b_).abs().max()))


def test_noalloc_scratch_limit(ldc):
    """A problem whose workspace exceeds the scratch is refused before any launch."""
    import torch
    T, H, d = 65536, 6, 128
    need = ldc.workspace_bytes(ldc.LDC_BF16, T, H, d, 112)
    assert need > ldc.noalloc_max_workspace()  # without saved state it does not fit
    w = wl.make_workload(T, H, d, dtype="bf16", seed=66, docs=("geometric", 1024))
    x = w.torch_inputs("cuda", with_do=True)
    args = (x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"])
    out = grads_like(torch, T, H, d)
    with pytest.raises(ldc.LDCError) as ei:
        ldc.bwd_noalloc(*args, None, x["do"], out, window=w.window, scale=w.scale)
    assert ei.value.status == 8
    torch.cuda.synchronize()
    assert all(bool(torch.isnan(t).all()) for t in out)  # nothing was written
