"""Host-side tests of the MUDD mixing C ABI (include/mudd.h).  No GPU needed:
every call here fails validation, or is a T == 0 no-op, before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

import dynamic_head_composition_amd as ldc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mudd.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ldc.LIB_PATH), reason="libldc.so not built")

A = 1 << 20  # fake 16-byte aligned device address, never dereferenced here
OK, NULL, SHAPE, DTYPE, ALIGN = 0, 1, 2, 3, 4


def ptrs(vals):
    arr = (ctypes.c_void_p * len(vals))()
    for i, v in enumerate(vals):
        arr[i] = v
    return arr


def fwd(dtype=0, T=8, dm=768, W=4, J=13, xs=None, a=A, ys=None):
    lib = ldc.load_library()
    xs = ptrs([A + 4096 * i for i in range(J)]) if xs is None else xs
    ys = ptrs([A + 65536 * (i + 1) for i in range(W)]) if ys is None else ys
    return lib.mudd_fwd(dtype, T, dm, W, J, xs, a, ys, None)


def bwd(dtype=0, T=8, dm=768, W=4, J=13, xs=None, a=A, dys=None, dxs=None, da=A):
    lib = ldc.load_library()
    xs = ptrs([A + 4096 * i for i in range(J)]) if xs is None else xs
    dys = ptrs([A + 65536 * (i + 1) for i in range(W)]) if dys is None else dys
    dxs = ptrs([A + 1048576 * (i + 1) for i in range(J)]) if dxs is None else dxs
    return lib.mudd_bwd(dtype, T, dm, W, J, xs, a, dys, dxs, da, None)


def test_header_declares_exported_symbols():
    names = sorted(set(re.findall(r"^\s*int\s+(mudd_\w+)\s*\(", open(HEADER).read(), re.M)))
    assert names == ["mudd_bwd", "mudd_fwd"]
    out = subprocess.run(["nm", "-D", "--defined-only", ldc.LIB_PATH], capture_output=True, text=True).stdout
    assert set(names) <= set(re.findall(r"\bT (mudd_\w+)", out))


def test_header_limits_match_binding():
    from dynamic_head_composition_amd import mudd
    text = open(HEADER).read()
    lim = {k: int(v) for k, v in re.findall(r"#define MUDD_MAX_(\w+) (\d+)", text)}
    assert (lim["STREAMS"], lim["WAYS"], lim["DIM"]) == (mudd.MAX_STREAMS, mudd.MAX_WAYS, mudd.MAX_DIM)


def test_zero_tokens_is_a_no_op():
    assert fwd(T=0) == OK
    assert bwd(T=0) == OK


@pytest.mark.parametrize("kw", [dict(dtype=2), dict(dtype=-1)])
def test_bad_dtype(kw):
    assert fwd(**kw) == DTYPE
    assert bwd(**kw) == DTYPE


@pytest.mark.parametrize("kw", [dict(T=-1), dict(W=0), dict(W=5), dict(J=0), dict(J=17),
                                dict(dm=0), dict(dm=3), dict(dm=6), dict(dm=16388),
                                dict(T=(1 << 40) // 768 + 1)])
def test_bad_shapes(kw):
    assert fwd(**kw) == SHAPE
    assert bwd(**kw) == SHAPE


def test_null_pointers():
    lib = ldc.load_library()
    assert lib.mudd_fwd(0, 8, 768, 1, 2, None, A, ptrs([A]), None) == NULL
    assert fwd(J=2, xs=ptrs([A, 0])) == NULL
    assert fwd(a=None) == NULL
    assert fwd(W=2, ys=ptrs([A, None])) == NULL
    assert bwd(da=None) == NULL
    assert bwd(W=1, dys=ptrs([0])) == NULL
    assert bwd(J=1, dxs=ptrs([0])) == NULL


def test_misaligned_pointers():
    assert fwd(J=2, xs=ptrs([A, A + 8])) == ALIGN
    assert fwd(a=A + 4) == ALIGN
    assert fwd(W=1, ys=ptrs([A + 2])) == ALIGN
    assert bwd(da=A + 4) == ALIGN
    assert bwd(W=1, dys=ptrs([A + 8])) == ALIGN
    assert bwd(J=1, dxs=ptrs([A + 12])) == ALIGN
