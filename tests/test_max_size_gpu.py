"""The largest stream the C ABI accepts at the GPT-2 small head shape (6 heads of
128): T*H*d + 512*H*d must stay below 2^31 elements, so T = 2,795,690 tokens
(4.3 GB per bf16 tensor, ~55 GB of device memory for one forward and backward,
a ragged last tile).  One size more is rejected.  Inputs are drawn on the GPU
from a seeded generator; three 512-token slices (first, middle, last) are
copied back with their window halo and checked against the fp64 oracle at the
bf16 bar, so every index and byte offset near the limit is exercised."""
import numpy as np
import pytest

from oracle import ldc_oracle as orc
from tests.helpers import assert_close, to_np

pytestmark = pytest.mark.gpu

H, D, W = 6, 128, 112
T_MAX = ((1 << 31) - 1 - 512 * H * D) // (H * D)
SLICE = 512


def test_limit_is_the_abi_limit(ldc):
    assert ldc.saved_bytes(ldc.LDC_BF16, T_MAX, H, D, W) > 0
    assert ldc.saved_bytes(ldc.LDC_BF16, T_MAX + 1, H, D, W) == 0  # rejected: LDC_ERR_SHAPE


def test_max_size_fwd_bwd(ldc):
    import torch
    T = T_MAX
    print(f"max-size case: T={T} H={H} d={D}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(2024)

    def normal(shape, std=1.0):
        x = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)
        return x.mul_(std)

    q = normal((T, H, D)).to(torch.bfloat16)
    k = normal((T, H, D)).to(torch.bfloat16)
    v = normal((T, H, D)).to(torch.bfloat16)
    do = normal((T, H, D)).to(torch.bfloat16)
    c = normal((T, H), 0.5)
    g = torch.rand((T, H), generator=gen, device="cuda", dtype=torch.float32).add_(0.5)
    starts = torch.rand((T,), generator=gen, device="cuda") < 1.0 / 1024
    doc = starts.to(torch.int32).cumsum_(0).to(torch.int32)
    scale = 1.0 / np.sqrt(D)

    o, saved = ldc.fwd(q, k, v, c, g, doc, window=W, scale=scale, save=True)
    grads = ldc.bwd(q, k, v, c, g, doc, saved, do, window=W, scale=scale)
    torch.cuda.synchronize()
    res = dict(zip(("o", "dq", "dk", "dv", "dc", "dg"), (o,) + tuple(grads)))
    for key, val in res.items():
        assert bool(torch.isfinite(val).all()), key

    for a in (0, T // 2 + 77, T - SLICE):
        lo, hi = max(0, a - W), min(T, a + SLICE + W)  # the slice and its window halo
        win = {name: to_np(t[lo:hi]).astype(np.float64) for name, t in
               (("q", q), ("k", k), ("v", v), ("do", do), ("c", c), ("g", g))}
        dwin = doc[lo:hi].cpu().numpy()
        r0, r1 = a - lo, a - lo + SLICE
        ref_o = orc.forward_slice(win["q"], win["k"], win["v"], win["c"], win["g"], dwin, r0, r1,
                                  window=W, scale=scale)
        assert_close(f"o[{a}:{a + SLICE}]", to_np(o[a:a + SLICE]), ref_o, "bf16")
        ref = orc.backward_slice(win["q"], win["k"], win["v"], win["c"], win["g"], dwin, win["do"],
                                 r0, r1, window=W, scale=scale)
        for key, r in zip(("dq", "dk", "dv", "dc", "dg"), ref):
            assert_close(f"{key}[{a}:{a + SLICE}]", to_np(res[key][a:a + SLICE]), r, "bf16")
