#!/usr/bin/env python3
"""Throughput of the Lightweight DC layer (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]
    python bench.py --workload mudd     # MUDD layer mixing (fwd + bwd) instead

A step is one forward pass and one backward pass of the layer over the whole
synthetic token stream of the workload (inputs resident in HBM before timing):
ldc_fwd, then ldc_bwd as its two kernels ldc_bwd_q and ldc_bwd_kv, each timed
with HIP events on the stream it runs on.  Rank 0 prints one JSON line.
The default warm-up (100 untimed steps, ~50 ms) brings the GPU from idle to
its sustained clocks before the timed steps.

The workload (default: the GPT-2 small layer, T=65536 flattened tokens, 6
heads of dim 128, window 112, documents of geometric length with mean 1024)
is seeded and synthetic; it stands in for the FineWeb token stream the
speedrun trains on.  The CPU baseline times the fp64 oracle on the host cores
over a bounded leading part of the same stream.

With --workload mudd the step is one MUDD mix forward and backward
(mudd_fwd + mudd_bwd) over a GPT-2 small token stream (65,536 tokens, model
dim 768, 13 layer streams, 4 ways), reported in the same format.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA
MFMA_F32_PEAK_TFLOPS = 157.3
METRIC = "LDC attention fwd+bwd tokens/s on 1 MI355X (GPT-2-small shape); % MFMA peak"
KERNELS = ("ldc_fwd", "ldc_bwd_q", "ldc_bwd_kv")
SOURCES = ("ldc_device.hpp", "ldc_pipeline.hpp", "ldc_fwd.hip", "ldc_bwd.hip", "ldc_internal.h")
MUDD_METRIC = "MUDD layer mixing fwd+bwd tokens/s on 1 MI355X (GPT-2-small stream)"
MUDD_KERNELS = ("mudd_fwd", "mudd_bwd")
MUDD_SOURCES = ("mudd.hip", "mudd_internal.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def valid_pairs(doc: np.ndarray, window: int) -> int:
    """(query, key) pairs admitted by the window and the document cut, for a
    stream whose documents are contiguous runs."""
    T = len(doc)
    starts = np.ones(T, dtype=bool)
    starts[1:] = doc[1:] != doc[:-1]
    idx = np.arange(T)
    first = np.maximum.accumulate(np.where(starts, idx, 0))
    return int(np.minimum(idx - first + 1, window).sum())


def algorithmic_bytes_per_token(H: int, d: int, elem: int) -> dict:
    """Compulsory HBM bytes per token of each kernel: every input it must read
    and every output it must write, once.  The saved state of the forward is
    512 B/token of shared-map band (2,048 four-byte words per 16 tokens) plus
    8 B per (token, head) of softmax statistics; the backward workspace holds
    the dPbar band (512 B/token)."""
    row = H * d
    ch = 4 * H    # one float per (token, head)
    band = 512    # shared-map or dPbar band
    stats = 2 * ch
    return {
        # q, k, v, c, g, doc in; o (fp32), saved band + statistics out
        "ldc_fwd": 3 * row * elem + 2 * ch + 4 + row * 4 + band + stats,
        # q, k, v, dO, c, g, doc, saved band + statistics in; dq, dc, dg, dPbar band out
        "ldc_bwd_q": 4 * row * elem + 2 * ch + 4 + band + stats + row * 4 + 2 * ch + band,
        # q, k, dO, c, g, dc, statistics, doc, both bands in; dk, dv out
        "ldc_bwd_kv": 3 * row * elem + 3 * ch + stats + 4 + 2 * band + 2 * row * 4,
    }


def source_digest(files=SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "dynamic_head_composition_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, files=SOURCES):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when it is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload, {}).get(kernel)
    if not ent or ent.get("source_digest") != source_digest(files):
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(w, budget_s: float, chunk: int = 8192):
    """Time the fp64 oracle (forward + backward) on leading slices of the
    stream until `budget_s` seconds of CPU work or the whole stream."""
    from oracle import ldc_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    done = 0
    t0 = time.perf_counter()
    while done < w.T and time.perf_counter() - t0 < budget_s:
        lo, hi = done, min(w.T, done + chunk)
        orc.forward_slice(w.q, w.k, w.v, w.c, w.g, w.doc, lo, hi, window=w.window, scale=w.scale)
        orc.backward_slice(w.q, w.k, w.v, w.c, w.g, w.doc, w.do, lo, hi, window=w.window, scale=w.scale)
        done = hi
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 oracle forward+backward over tokens [0, {done}) of the same stream, "
                      f"in {chunk}-token slices with their window halo; {el:.1f} s"}


def copy_probe(mib: int) -> None:
    """One plain device copy of `mib` MiB: a kernel of known traffic against
    which rocprofv3's HBM byte counters are calibrated."""
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def mudd_bytes_per_token(dm: int, W: int, J: int, elem: int) -> dict:
    """Compulsory HBM bytes per token of the two MUDD kernels."""
    return {
        # J streams and the W x J weights in; W float32 mixes out
        "mudd_fwd": J * dm * elem + W * J * 4 + W * dm * 4,
        # J streams, W upstream gradients and the weights in; J float32 stream
        # gradients and the W x J weight gradients out
        "mudd_bwd": (J + W) * dm * elem + W * J * 4 + J * dm * 4 + W * J * 4,
    }


def mudd_cpu_baseline(w, budget_s: float, chunk: int = 2048):
    """Time the fp64 MUDD oracle (forward + backward) on leading row slices
    until `budget_s` seconds of CPU work or the whole stream."""
    from oracle import mudd_oracle as mo
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    done = 0
    t0 = time.perf_counter()
    while done < w.T and time.perf_counter() - t0 < budget_s:
        lo, hi = done, min(w.T, done + chunk)
        xs = [x[lo:hi] for x in w.xs]
        mo.forward(xs, w.a[lo:hi])
        mo.backward(xs, w.a[lo:hi], [d[lo:hi] for d in w.dys])
        done = hi
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 oracle forward+backward over tokens [0, {done}) of the same stream, "
                      f"in {chunk}-token slices; {el:.1f} s"}


def bench_mudd(args):
    import torch
    import dynamic_head_composition_amd as ldc
    from dynamic_head_composition_amd import mudd
    from dynamic_head_composition_amd import workloads as wl

    ldc.load_library()  # fails loudly when the HIP library is missing
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    cfg = dict(wl.MUDD_BENCH)
    if args.tokens:
        cfg["T"] = args.tokens
    log(f"generating MUDD workload {cfg} ...")
    w = wl.make_mudd_workload(**cfg)
    xs, a, dys = w.torch_inputs("cuda")
    T, dm, W, J = w.T, w.dm, w.W, w.J
    elem = 2 if w.dtype == "bf16" else 4
    f32 = dict(dtype=torch.float32, device="cuda")
    ys = [torch.empty((T, dm), **f32) for _ in range(W)]
    dxs = [torch.empty((T, dm), **f32) for _ in range(J)]
    da = torch.empty((T, W, J), **f32)

    def step(evs=None):
        if evs:
            evs[0].record()
        mudd.fwd(xs, a, out=ys)
        if evs:
            evs[1].record()
        mudd.bwd(xs, a, dys, out=(dxs, da))
        if evs:
            evs[2].record()

    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if not all(bool(torch.isfinite(t).all()) for t in ys + dxs + [da]):
        raise SystemExit("non-finite outputs")
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kernel_ms = {kn: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)]))
                 for j, kn in enumerate(MUDD_KERNELS)}
    bpt = mudd_bytes_per_token(dm, W, J, elem)
    per_kernel = {kn: {"avg_us": round(kernel_ms[kn] * 1e3, 2), "alg_bytes_per_launch": bpt[kn] * T,
                       "alg_GBps": round(bpt[kn] * T / (kernel_ms[kn] * 1e-3) / 1e9, 1)}
                  for kn in MUDD_KERNELS}
    dominant = max(MUDD_KERNELS, key=lambda kn: kernel_ms[kn])
    achieved = bpt[dominant] * T / (kernel_ms[dominant] * 1e-3) / 1e9
    value = T / (ms_per_step * 1e-3)
    ceiling_tps = HBM_PEAK_GBPS * 1e9 / sum(bpt.values())
    line = {
        "metric": MUDD_METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": T, "model_dim": dm, "ways": W, "streams": J,
                   "recipe": w.recipe, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(dominant, w.name, MUDD_SOURCES)},
        "step_hbm_ceiling_tokens_per_s": round(ceiling_tps, 1),
        "step_roofline_frac": round(value / ceiling_tps, 4),
        "kernels": per_kernel,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        line["cpu_baseline"] = mudd_cpu_baseline(w, args.cpu_budget)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the first milliseconds of load after an idle GPU run at lower clocks
    # (measured: 5 warm-up steps read ~10% below 100); 100 steps take ~50 ms
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", type=int, default=2, help="workload index (2 = GPT-2 small layer fwd+bwd)")
    ap.add_argument("--workload", choices=("ldc", "mudd"), default="ldc",
                    help="ldc: the Lightweight DC layer (default); mudd: MUDD layer mixing")
    ap.add_argument("--tokens", type=int, default=None, help="truncate the stream (quick runs only)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before timing, copy a buffer of this many MiB once (a plain copy kernel of "
                         "known traffic, to calibrate HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)
    if args.workload == "mudd":
        return bench_mudd(args)

    import torch
    import dynamic_head_composition_amd as ldc
    from dynamic_head_composition_amd import workloads as wl

    ldc.load_library()  # fails loudly when the HIP library is missing
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")

    log(f"generating workload {args.config} ...")
    w = wl.config_workload(args.config, T=args.tokens)
    x = w.torch_inputs("cuda")
    T, H, d = w.T, w.H, w.d
    elem = 2 if w.dtype == "bf16" else 4
    f32 = dict(dtype=torch.float32, device="cuda")
    o = torch.empty((T, H, d), **f32)
    grads = (torch.empty((T, H, d), **f32), torch.empty((T, H, d), **f32),
             torch.empty((T, H, d), **f32), torch.empty((T, H), **f32), torch.empty((T, H), **f32))
    code = ldc.LDC_BF16 if w.dtype == "bf16" else ldc.LDC_F32
    ws = torch.empty(max(16, ldc.workspace_bytes(code, T, H, d, w.window)), dtype=torch.uint8, device="cuda")
    saved = torch.empty(max(16, ldc.saved_bytes(code, T, H, d, w.window)), dtype=torch.uint8, device="cuda")
    ins = (x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"])

    def step(evs=None):
        if evs:
            evs[0].record()
        ldc.fwd(*ins, window=w.window, scale=w.scale, out=o, saved=saved)
        if evs:
            evs[1].record()
        ldc.bwd(*ins, saved, x["do"], window=w.window, scale=w.scale, out=grads, workspace=ws, part="q")
        if evs:
            evs[2].record()
        ldc.bwd(*ins, saved, x["do"], window=w.window, scale=w.scale, out=grads, workspace=ws, part="kv")
        if evs:
            evs[3].record()

    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if not all(bool(torch.isfinite(t).all()) for t in (o,) + grads):
        raise SystemExit("non-finite outputs")

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kernel_ms = {kname: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)]))
                 for j, kname in enumerate(KERNELS)}
    pairs = valid_pairs(w.doc, w.window)
    total_flops = 14.0 * H * d * pairs
    bpt = algorithmic_bytes_per_token(H, d, elem)
    per_kernel = {}
    for kname in KERNELS:
        sec = kernel_ms[kname] * 1e-3
        per_kernel[kname] = {"avg_us": round(kernel_ms[kname] * 1e3, 2),
                             "alg_bytes_per_launch": bpt[kname] * T,
                             "alg_GBps": round(bpt[kname] * T / sec / 1e9, 1)}
    dominant = max(KERNELS, key=lambda kname: kernel_ms[kname])
    dom_sec = kernel_ms[dominant] * 1e-3
    achieved = bpt[dominant] * T / dom_sec / 1e9
    traffic = measured_traffic(dominant, w.name)
    value = T / (ms_per_step * 1e-3)
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    alg_tflops = total_flops / (ms_per_step * 1e-3) / 1e12
    alg_bytes_step = sum(bpt[kn] for kn in KERNELS) * T
    ceiling_tps = HBM_PEAK_GBPS * 1e9 / (alg_bytes_step / T)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": T, "heads": H, "head_dim": d, "window": w.window,
                   "recipe": w.recipe, "valid_pairs": pairs, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic},
        "mfma_peak_frac": round(alg_tflops / mfma_peak, 5),
        "alg_TFLOPs": round(alg_tflops, 2),
        "step_hbm_ceiling_tokens_per_s": round(ceiling_tps, 1),
        "step_roofline_frac": round(value / ceiling_tps, 4),
        "kernels": per_kernel,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
