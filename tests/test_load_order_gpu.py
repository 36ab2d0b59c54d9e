"""The library loaded through the binding before the caller imports torch
(as build() does): the binding imports torch first, so the launches use the
HIP runtime that owns torch's streams and memory.  Loading libldc.so ahead of
torch's runtime made every launch fail with LDC_ERR_HIP.  Runs in a fresh
process, since the order only matters at the first load."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys
sys.path.insert(0, sys.argv[1])
import dynamic_head_composition_amd as ldc
ldc.load_library()                      # before this script imports torch
import numpy as np
import torch
from dynamic_head_composition_amd import workloads as wl
from oracle import ldc_oracle as orc
w = wl.make_workload(200, 2, 64, dtype="bf16", seed=3, docs=("geometric", 40))
x = w.torch_inputs("cuda:0", with_do=False)
o = ldc.fwd(x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"], window=w.window, scale=w.scale)
torch.cuda.synchronize()
ref = orc.forward(w.q, w.k, w.v, w.c, w.g, w.doc, window=w.window, scale=w.scale)
err = float(np.max(np.abs(o.cpu().numpy().astype(np.float64) - ref)))
print("max_abs", err, flush=True)
assert err <= 2e-2
"""


def test_library_loaded_before_torch():
    out = subprocess.run([sys.executable, "-c", SCRIPT, ROOT], capture_output=True, text=True, timeout=240)
    print(out.stdout[-2000:], out.stderr[-2000:])
    assert out.returncode == 0
