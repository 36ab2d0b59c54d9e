"""Host-side tests of the C ABI (no GPU needed: validation precedes any HIP call)."""
import ctypes
import os
import re
import subprocess

import pytest

import dynamic_head_composition_amd as ldc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ldc.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ldc.LIB_PATH), reason="libldc.so not built")

A = 1 << 20  # a fake, 16-byte aligned address; never dereferenced by these tests


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(ldc_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    lib = ldc.load_library()
    names = declared_functions()
    assert names == ["ldc_bwd", "ldc_bwd_kv", "ldc_bwd_noalloc", "ldc_bwd_noalloc_max_workspace",
                     "ldc_bwd_q", "ldc_bwd_workspace_bytes", "ldc_fwd", "ldc_saved_bytes",
                     "ldc_status_str", "ldc_version"]
    for nm in names:
        assert hasattr(lib, nm)
    out = subprocess.run(["nm", "-D", "--defined-only", ldc.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (ldc_\w+)", out))
    assert set(names) <= exported


def test_version_and_status_strings():
    assert ldc.version() == 10000
    for code in range(9):
        assert ldc.status_str(code).startswith("LDC_")
    assert "unknown" in ldc.status_str(99)


def room(n):
    return (n + 255) // 256 * 256


def test_workspace_and_saved_bytes():
    band = 4096 * 2048 * 4  # 4,096 blocks of 16 queries x 2,048 words
    saved = band + 65536 * 6 * 8
    assert ldc.saved_bytes(ldc.LDC_BF16, 65536, 6, 128, 112) == saved
    # room for the recomputed saved state (when the caller passes none) + the dPbar band
    assert ldc.workspace_bytes(ldc.LDC_BF16, 65536, 6, 128, 112) == room(saved) + band
    assert ldc.workspace_bytes(ldc.LDC_F32, 17, 3, 16, 5) == room(2 * 8192 + 17 * 3 * 8) + 2 * 8192
    assert ldc.saved_bytes(ldc.LDC_F32, 17, 2, 16, 112) == 2 * 2048 * 4 + 17 * 2 * 8
    assert ldc.workspace_bytes(ldc.LDC_BF16, 0, 6, 128, 112) == 0
    assert ldc.workspace_bytes(ldc.LDC_BF16, 10, 6, 32, 112) == 0  # unsupported -> 0
    assert ldc.workspace_bytes(ldc.LDC_BF16, 10, 6, 16, 112) == room(8192 + 10 * 6 * 8) + 8192
    # windows above 113 keys: bands of 10 key blocks (2,560 words per 16-query block)
    wide = 4096 * 2560 * 4
    assert ldc.saved_bytes(ldc.LDC_BF16, 65536, 6, 128, 128) == wide + 65536 * 6 * 8
    assert ldc.saved_bytes(ldc.LDC_BF16, 65536, 6, 128, 114) == wide + 65536 * 6 * 8
    assert ldc.saved_bytes(ldc.LDC_BF16, 65536, 6, 128, 113) == band + 65536 * 6 * 8
    assert ldc.workspace_bytes(ldc.LDC_F32, 17, 3, 64, 120) == room(2 * 10240 + 17 * 3 * 8) + 2 * 10240
    assert ldc.saved_bytes(ldc.LDC_F32, 17, 3, 128, 120) == 0       # f32 d=128: window <= 113


def fwd_call(dtype=ldc.LDC_BF16, T=256, H=6, d=128, window=112, ptrs=None, saved=None, saved_bytes=0,
             scale=0.1):
    lib = ldc.load_library()
    p = ptrs or [A] * 7
    return lib.ldc_fwd(dtype, T, H, d, window, scale, *p, saved, saved_bytes, None)


def bwd_call(dtype=ldc.LDC_BF16, T=256, H=6, d=128, window=112, ptrs=None, ws=A, ws_bytes=None,
             saved=A, saved_bytes=None, entry="ldc_bwd", scale=0.1):
    lib = ldc.load_library()
    p = ptrs or [A] * 12
    if ws_bytes is None:
        ws_bytes = ldc.workspace_bytes(dtype, T, H, d, window)
    if saved_bytes is None:
        saved_bytes = ldc.saved_bytes(dtype, T, H, d, window)
    return getattr(lib, entry)(dtype, T, H, d, window, scale, *p[:6], saved, saved_bytes, *p[6:],
                               ws, ws_bytes, None)


def bwd_noalloc_call(dtype=ldc.LDC_BF16, T=256, H=6, d=128, window=112, ptrs=None, saved=A,
                     saved_bytes=None, scale=0.1):
    lib = ldc.load_library()
    p = ptrs or [A] * 12
    if saved_bytes is None:
        saved_bytes = ldc.saved_bytes(dtype, T, H, d, window)
    return lib.ldc_bwd_noalloc(dtype, T, H, d, window, scale, *p[:6], saved, saved_bytes, *p[6:], None)


def bwd_q_call(**kw):
    return bwd_call(entry="ldc_bwd_q", **kw)


def bwd_kv_call(**kw):
    return bwd_call(entry="ldc_bwd_kv", **kw)


@pytest.mark.parametrize("call", [fwd_call, bwd_call, bwd_q_call, bwd_kv_call, bwd_noalloc_call])
def test_validation_errors(call):
    assert call(dtype=2) == 3                      # LDC_ERR_DTYPE
    assert call(T=-1) == 2                         # LDC_ERR_SHAPE
    assert call(H=0) == 2
    assert call(window=0) == 2
    assert call(window=129) == 2
    assert call(dtype=ldc.LDC_F32, d=128, window=114) == 5  # no LDS for f32 rows of 128 there
    assert call(T=1 << 31) == 2                    # too many rows
    assert call(scale=0.0) == 2                    # scale must be positive and finite
    assert call(scale=-0.5) == 2
    assert call(scale=float("inf")) == 2
    assert call(scale=float("nan")) == 2
    assert call(d=32) == 5                         # LDC_ERR_UNSUPPORTED
    assert call(d=256) == 5
    nptr = 7 if call is fwd_call else 12
    for i in range(nptr):
        ptrs = [A] * nptr
        ptrs[i] = None
        assert call(ptrs=ptrs) == 1                # LDC_ERR_NULL
        ptrs[i] = A + 8
        assert call(ptrs=ptrs) == 4                # LDC_ERR_ALIGN


@pytest.mark.parametrize("entry", ["ldc_bwd", "ldc_bwd_q", "ldc_bwd_kv"])
def test_bwd_workspace_errors(entry):
    band = ldc.workspace_bytes(ldc.LDC_BF16, 256, 6, 128, 112) - room(ldc.saved_bytes(ldc.LDC_BF16, 256, 6, 128, 112))
    assert band == 16 * 8192
    assert bwd_call(ws=None, entry=entry) == 6
    assert bwd_call(ws_bytes=100, entry=entry) == 6
    assert bwd_call(ws_bytes=band - 16, entry=entry) == 6      # saved given: the band is enough
    assert bwd_call(ws=A + 4, entry=entry) == 4
    assert bwd_call(saved=None, ws_bytes=band, entry=entry) == 6  # no saved state: room for it too
    assert bwd_call(saved_bytes=100, entry=entry) == 6
    assert bwd_call(saved=A + 4, entry=entry) == 4


def test_noalloc_scratch_limit():
    """ldc_bwd_noalloc refuses, before any HIP call, a problem whose workspace
    exceeds its 64 MiB static scratch; other errors come first."""
    lib = ldc.load_library()
    assert lib.ldc_bwd_noalloc_max_workspace() == 64 << 20
    # with saved state the workspace is the dPbar band, 512 bytes per token
    assert bwd_noalloc_call(T=131073, H=1, d=16, dtype=ldc.LDC_F32) == 8       # LDC_ERR_SCRATCH
    # without, it also holds the recomputed state
    assert bwd_noalloc_call(T=65536, H=6, saved=None, saved_bytes=0) == 8
    assert bwd_noalloc_call(T=131073, H=1, d=16, dtype=ldc.LDC_F32, saved_bytes=100) == 6
    assert bwd_noalloc_call(T=131073, H=1, d=16, dtype=ldc.LDC_F32, saved=A + 4) == 4
    assert lib.ldc_bwd_noalloc(0, 0, 6, 128, 112, 0.1, *([None] * 6), None, 0, *([None] * 6), None) == 0
    assert "static scratch" in ldc.status_str(8)


def test_fwd_saved_errors():
    need = ldc.saved_bytes(ldc.LDC_BF16, 256, 6, 128, 112)
    assert fwd_call(saved=A, saved_bytes=need - 16) == 6
    assert fwd_call(saved=A + 4, saved_bytes=need) == 4


def test_empty_stream_is_a_noop():
    # T == 0 returns before any HIP call, even with NULL pointers
    lib = ldc.load_library()
    assert lib.ldc_fwd(0, 0, 6, 128, 112, 0.1, *([None] * 7), None, 0, None) == 0
    assert lib.ldc_bwd(0, 0, 6, 128, 112, 0.1, *([None] * 6), None, 0, *([None] * 6), None, 0, None) == 0


def test_oracle_and_product_share_no_code():
    pkg = os.path.join(ROOT, "dynamic_head_composition_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, re.M), f
                assert "oracle/" not in text, f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            text = open(os.path.join(ROOT, "oracle", f), encoding="utf-8").read()
            assert "dynamic_head_composition_amd" not in text, f
