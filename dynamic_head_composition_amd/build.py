"""Build the HIP library libldc.so (every kernel of the package) in-tree for gfx950.

    python -m dynamic_head_composition_amd.build [--verbose]

Every HIP source is compiled with packed-fp32 instructions disabled
(`-target-feature -packed-fp32-ops`); the library is written next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libldc.so")
SOURCES = ["ldc_fwd.hip", "ldc_bwd.hip", "ldc_api.cpp", "dcmha.hip", "dcmha_api.cpp", "cg.hip", "cg_api.cpp", "mudd.hip", "mudd_api.cpp", "fused.hip", "fused_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if p and os.path.exists(p):
            return p
    return "hipcc"


def flags():
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument"]


def build(verbose: bool = False, jobs: int = 3) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        objs.append(obj)
        lang = [] if src.endswith(".hip") else ["-x", "hip"]
        cmd = [hipcc(), *flags(), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0), verbose)
    for p in procs:
        _wait(p, verbose)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    out = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if out.returncode != 0:
        raise RuntimeError("link failed:\n" + out.stdout)
    os.replace(tmp, LIB)
    return LIB


def _wait(item, verbose):
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    if p.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{text}")
    if verbose and text.strip():
        print(text, flush=True)


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
