"""Host-side tests of the generator's C ABI (validation precedes any HIP call)."""
import os
import re
import subprocess

import pytest

import dynamic_head_composition_amd as ldc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.skipif(not os.path.exists(ldc.LIB_PATH), reason="libldc.so not built")
A = 1 << 20


def test_exports_every_declared_symbol():
    text = open(os.path.join(ROOT, "include", "ldc_cg.h")).read()
    names = sorted(set(re.findall(r"^\s*(?:int|size_t)\s+(ldc_cg_\w+)\s*\(", text, re.M)))
    assert names == ["ldc_cg_bwd", "ldc_cg_bwd_workspace_bytes", "ldc_cg_fwd"]
    out = subprocess.run(["nm", "-D", "--defined-only", ldc.LIB_PATH], capture_output=True, text=True).stdout
    assert set(names) <= set(re.findall(r"\bT (ldc_cg_\w+)", out))


def test_workspace_bytes():
    from dynamic_head_composition_amd import cg
    assert cg.workspace_bytes(ldc.LDC_BF16, 65536, 768, 6) == 256 * 16 * 768 * 4
    assert cg.workspace_bytes(ldc.LDC_BF16, 300, 768, 6) == 2 * 16 * 768 * 4
    assert cg.workspace_bytes(ldc.LDC_BF16, 0, 768, 6) == 0
    assert cg.workspace_bytes(ldc.LDC_F32, 10, 1024, 6) == 0   # f32: dm <= 768
    assert cg.workspace_bytes(ldc.LDC_BF16, 10, 96, 6) == 0    # dm a multiple of 64


def test_validation_errors():
    lib = ldc.load_library()
    fwd = lambda dtype=0, T=100, dm=768, H=6, p=None: lib.ldc_cg_fwd(dtype, T, dm, H, *(p or [A] * 5), None)
    assert fwd(dtype=2) == 3
    assert fwd(T=-1) == 2
    assert fwd(H=0) == 2
    assert fwd(H=9) == 5
    assert fwd(dm=96) == 5
    assert fwd(dm=1088) == 5
    assert fwd(dtype=1, dm=832) == 5
    for i in range(5):
        p = [A] * 5
        p[i] = None
        assert fwd(p=p) == 1
        p[i] = A + 4
        assert fwd(p=p) == 4
    assert lib.ldc_cg_fwd(0, 0, 768, 6, *([None] * 5), None) == 0   # empty stream: no-op
    bwd = lambda ws=A, wsb=1 << 30, p=None: lib.ldc_cg_bwd(0, 100, 768, 6, *(p or [A] * 8), ws, wsb, None)
    assert bwd(ws=None) == 6
    assert bwd(wsb=100) == 6
    assert bwd(ws=A + 4) == 4
    for i in range(8):
        p = [A] * 8
        p[i] = None
        assert bwd(p=p) == 1
