"""Host-side tests of the fused block's C ABI (validation precedes any HIP call)."""
import os
import re
import subprocess

import pytest

import dynamic_head_composition_amd as ldc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ldc_fused.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ldc.LIB_PATH), reason="libldc.so not built")

A = 1 << 20  # fake aligned address, never dereferenced here


def test_exports_every_declared_symbol():
    names = sorted(set(re.findall(r"^\s*(?:int|size_t)\s+(ldc_\w+)\s*\(", open(HEADER).read(), re.M)))
    assert names == ["ldc_fused_fwd", "ldc_fused_fwd_workspace_bytes", "ldc_main_attention_fwd",
                     "ldc_main_attention_workspace_bytes"]
    out = subprocess.run(["nm", "-D", "--defined-only", ldc.LIB_PATH], capture_output=True, text=True).stdout
    assert set(names) <= set(re.findall(r"\bT (ldc_\w+)", out))


def test_workspace_sizes():
    from dynamic_head_composition_amd import fused as fz
    room = lambda n: (n + 255) // 256 * 256
    # run-start block summaries, one run start per token, then the item
    # order: a histogram and cursors of 1024 classes and one int per tile
    runs = lambda T: room((T + 1023) // 1024 * 4) + room(4 * T) + 4 * (2048 + (T + 127) // 128)
    for T, H, d in ((65536, 6, 128), (1, 1, 64), (1000, 7, 64)):
        saved = ldc.saved_bytes(ldc.LDC_BF16, T, H, d)
        assert saved > 0
        assert fz.workspace_bytes(ldc.LDC_BF16, T, H, d) == room(saved) + runs(T)
        assert fz.main_workspace_bytes(T) == runs(T)
    assert fz.workspace_bytes(ldc.LDC_BF16, 0, 6, 128) == 0
    assert fz.workspace_bytes(ldc.LDC_F32, 100, 6, 64) == 0      # bf16 only
    assert fz.workspace_bytes(ldc.LDC_BF16, 100, 6, 128, 129) == 0
    assert fz.main_workspace_bytes(0) == 0


def ws_of(T=256, H=6, d=128, window=112):
    from dynamic_head_composition_amd import fused as fz
    return fz.workspace_bytes(ldc.LDC_BF16, T, H, d, window)


def fused(dtype=ldc.LDC_BF16, T=256, H=6, d=128, window=112, scale=0.1, ptrs=None, ws=A, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = ws_of(T, H, d, window) if dtype == ldc.LDC_BF16 and 0 < T < 1 << 20 else 1 << 40
    return ldc.load_library().ldc_fused_fwd(dtype, T, H, d, window, scale, *(ptrs or [A] * 7), ws, ws_bytes,
                                            None)


def main(dtype=ldc.LDC_BF16, T=256, H=6, d=128, scale=0.1, ptrs=None, ws=A, ws_bytes=1 << 30):
    return ldc.load_library().ldc_main_attention_fwd(dtype, T, H, d, scale, *(ptrs or [A] * 5), ws, ws_bytes,
                                                     None)


def test_fused_validation():
    assert fused(dtype=2) == 3                      # not a dtype
    assert fused(T=-1) == 2
    assert fused(H=0) == 2
    assert fused(window=0) == 2 and fused(window=129) == 2
    assert fused(scale=0.0) == 2 and fused(scale=float("inf")) == 2
    assert fused(T=1 << 24, H=6, d=128) == 2      # T*H*d beyond int32
    assert fused(dtype=ldc.LDC_F32, d=64) == 5    # bf16 only
    assert fused(d=16) == 5 and fused(d=96) == 5
    for i in range(7):
        p = [A] * 7
        p[i] = None
        assert fused(ptrs=p) == 1, i
        p[i] = A + 8
        assert fused(ptrs=p) == 4, i
    assert fused(ws=None) == 6
    assert fused(ws_bytes=ws_of() - 1) == 6
    assert fused(ws=A + 8) == 4
    assert fused(T=0, ptrs=[None] * 7, ws=None, ws_bytes=0) == 0     # empty: a no-op, nothing read


def test_main_validation():
    assert main(dtype=2) == 3
    assert main(T=-1) == 2 and main(H=0) == 2 and main(scale=-1.0) == 2
    assert main(dtype=ldc.LDC_F32, d=64) == 5 and main(d=32) == 5
    for i in range(5):
        p = [A] * 5
        p[i] = None
        assert main(ptrs=p) == 1, i
        p[i] = A + 4
        assert main(ptrs=p) == 4, i
    assert main(ws=None) == 6
    from dynamic_head_composition_amd import fused as fz
    assert main(ws_bytes=fz.main_workspace_bytes(256) - 1) == 6
    assert main(T=0, ptrs=[None] * 5, ws=None, ws_bytes=0) == 0


def test_python_binding_rejects_host_tensors():
    import torch
    from dynamic_head_composition_amd import fused as fz
    q = torch.zeros(8, 2, 64, dtype=torch.bfloat16)
    c = torch.zeros(8, 2)
    doc = torch.zeros(8, dtype=torch.int32)
    with pytest.raises(ValueError):
        fz.fwd(q, q, q, c, c, doc)
    with pytest.raises(ValueError):
        fz.main_fwd(q, q, q, doc)
