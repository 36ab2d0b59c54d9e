"""Host-side checks of the benchmark's accounting (CPU): the algorithmic bytes
per token of each pass (the layer's compulsory I/O, every tensor once), the
admitted-pair count against a brute-force count, the fused call's stage
count against a per-tile loop, and the one-GPU guard."""
import os
import subprocess
import sys

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_spec_bytes_per_token():
    # forward: Q, K, V (3 H d e) + C, G (8H) + doc (4) + O (H d e);
    # backward: Q, K, V, dO (4 H d e) + C, G (8H) + doc (4) + dQ, dK, dV fp32 (12 H d) + dC, dG (8H)
    assert bench.spec_bytes_per_token(6, 128, 2) == {"ldc_fwd": 6196, "ldc_bwd": 15460}
    assert bench.spec_bytes_per_token(12, 64, 2) == {"ldc_fwd": 6244, "ldc_bwd": 15556}
    assert bench.spec_bytes_per_token(2, 16, 4) == {"ldc_fwd": 4 * 2 * 16 * 4 + 16 + 4,
                                                     "ldc_bwd": 4 * 2 * 16 * 4 + 32 + 4 + 3 * 2 * 16 * 4}


def test_valid_pairs_brute_force():
    rng = np.random.default_rng(0)
    for T, window in ((1, 1), (50, 1), (300, 7), (700, 112), (257, 128)):
        lengths = rng.integers(1, 60, size=T)
        doc = np.repeat(np.arange(T), lengths)[:T].astype(np.int32)
        brute = sum(1 for t in range(T) for s in range(max(0, t - window + 1), t + 1) if doc[s] == doc[t])
        assert bench.valid_pairs(doc, window) == brute


def test_fused_design_bytes_counts_stages():
    rng = np.random.default_rng(1)
    T, H, d = 1500, 3, 64
    doc = np.repeat(np.arange(T), rng.integers(1, 700, size=T))[:T].astype(np.int32)
    stages = 0
    for q0 in range(0, T, 128):
        start = q0
        while start > 0 and doc[start - 1] == doc[q0]:
            start -= 1
        span = (q0 - 128) - start
        stages += (-(-span // 64) if span > 0 else 0) + 4
    row = H * d
    expect = (T * (2 * row * 2 + 8 * H + 4 + 512 + 8 * H) + T * 12
              + H * (stages * 2 * 64 + (-(-T // 128)) * 256) * d * 2
              + T * (row * 2 + 8 * H + 512 * H + row * 4))
    assert bench.fused_design_bytes(doc, H, d, 2) == expect


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert out.returncode == 2
    assert "one GPU" in out.stderr
