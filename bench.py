#!/usr/bin/env python3
"""Throughput of the Lightweight DC layer (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]
    python bench.py --workload mudd     # MUDD layer mixing (fwd + bwd) instead

A step is one forward pass and one backward pass of the layer over the whole
synthetic token stream of the workload (inputs resident in HBM before timing):
ldc_fwd, then ldc_bwd as its two kernels ldc_bwd_q and ldc_bwd_kv, each timed
with HIP events on the stream it runs on (median and interquartile range over
the timed steps).  Rank 0 prints one JSON line.

The roofline figures use the algorithmic bytes of each pass: the compulsory
I/O of the layer's definition, every input read once and every output written
once (forward 6,196 B/token, backward 15,460 B/token at 6 x 128 bf16).  The
bytes the kernels move as designed (float32 O, the saved state, the backward
workspace, the key-side kernel's second read of Q, K and dO) and the measured
HBM traffic (rocprofv3 counters) are reported beside them.
The default warm-up (100 untimed steps, ~50 ms) brings the GPU from idle to
its sustained clocks before the timed steps.

The workload (default: the GPT-2 small layer, T=65536 flattened tokens, 6
heads of dim 128, window 112, documents of geometric length with mean 1024)
is seeded and synthetic; it stands in for the FineWeb token stream the
speedrun trains on.  The CPU baseline times the fp64 oracle on the host cores
over a bounded leading part of the same stream.

With --workload dcmha the step is the full DCMHA composition layer (score and
weight compositions across heads, dcmha_fwd + dcmha_bwd_q + dcmha_bwd_kv) at
the same GPT-2 small shape, reported in the same format.

With --workload cg the step is the generator of the layer's weights (C = x WC,
G = x WG from the 768-wide hidden state) forward and backward.

With --workload fused the step is the attention block's forward with the
Lightweight DC layer fused into the main attention kernel (ldc_fused_fwd) on
the GPT-2 small forward workload; the unfused pair (ldc_main_attention_fwd,
then ldc_fwd) is timed beside it.

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
# the launches of each pass of the layer (a pass is one ABI call)
PASSES = {"ldc_fwd": ("ldc_fwd",), "ldc_bwd": ("ldc_bwd_q", "ldc_bwd_kv")}
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


def spec_bytes_per_token(H: int, d: int, elem: int) -> dict:
    """Algorithmic HBM bytes per token of each pass: the compulsory I/O of the
    layer's definition, every tensor once, O counted in the storage dtype.
    Forward: Q, K, V, C, G, doc in; O out.  Backward: Q, K, V, dO, C, G, doc
    in; dQ, dK, dV (float32), dC, dG out.  At 6 x 128 bf16: 6,196 and 15,460."""
    row = H * d
    return {"ldc_fwd": 3 * row * elem + 8 * H + 4 + row * elem,
            "ldc_bwd": 4 * row * elem + 16 * H + 4 + 3 * row * 4}


def design_bytes_per_token(H: int, d: int, elem: int) -> dict:
    """HBM bytes per token each kernel moves as designed: its inputs read once
    and its outputs written once, including the state the kernels pass each
    other (the shared-map band, 512 B/token, and the softmax statistics, 8 B
    per token and head, saved by the forward; the dPbar band, 512 B/token, in
    the backward workspace) and the key-side kernel's second read of Q, K and
    dO.  O and the gradients are float32."""
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


def measured_traffic(kernels, workload: str, files=SOURCES):
    """HBM bytes per launch summed over `kernels` (the launches of one pass),
    from the committed rocprofv3 counter summary, or None when an entry is
    missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    total = 0
    for kernel in kernels:
        ent = rec.get(workload, {}).get(kernel)
        if not ent or ent.get("source_digest") != source_digest(files):
            return None
        total += ent["bytes_per_launch"]
    return total


def host_cpu() -> dict:
    """CPU model and the cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "host_cores": len(os.sched_getaffinity(0))}


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


class TimingEvent:
    """A HIP event for timing only, recorded on torch's current stream (the
    stream the library's kernels are enqueued on).  Created with
    hipEventDisableSystemFence: recording it writes a timestamp without the
    system-scope fence (L2 write-back and invalidate) of a default event,
    which measured ~3 us per record at the GPT-2 small step and slowed the
    kernels after it.  elapsed_time(other) in ms, like torch's events."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes
            lib = ctypes.CDLL("libamdhip64.so")
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = lib
        return cls._hip

    def __init__(self):
        import ctypes
        self._ev = ctypes.c_void_p()
        st = self._lib().hipEventCreateWithFlags(ctypes.byref(self._ev), self.DISABLE_SYSTEM_FENCE)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")

    def record(self):
        import ctypes
        import torch
        st = self._lib().hipEventRecord(self._ev, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def elapsed_time(self, end) -> float:
        import ctypes
        ms = ctypes.c_float()
        st = self._lib().hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value

    def __del__(self):
        if self._hip is not None and getattr(self, "_ev", None):
            self._hip.hipEventDestroy(self._ev)


def stats_us(samples_ms) -> dict:
    """Median and interquartile range (µs) of per-step event times."""
    a = np.asarray(samples_ms, dtype=np.float64) * 1e3
    q1, med, q3 = np.percentile(a, [25, 50, 75])
    return {"median_us": round(float(med), 2), "iqr_us": round(float(q3 - q1), 2),
            "mean_us": round(float(a.mean()), 2)}


def cpu_baseline(w, budget_s: float, chunk: int = 8192, runs: int = 3):
    """Time the fp64 oracle (forward + backward) on leading slices of the
    stream: up to `runs` passes over the whole stream (the median is
    reported), or one pass over a leading part when a pass would exceed
    `budget_s` seconds."""
    from oracle import ldc_oracle as orc
    rates = []
    t_all = time.perf_counter()
    for _ in range(runs):
        done = 0
        t0 = time.perf_counter()
        while done < w.T and time.perf_counter() - t0 < budget_s:
            lo, hi = done, min(w.T, done + chunk)
            orc.forward_slice(w.q, w.k, w.v, w.c, w.g, w.doc, lo, hi, window=w.window, scale=w.scale)
            orc.backward_slice(w.q, w.k, w.v, w.c, w.g, w.doc, w.do, lo, hi, window=w.window,
                               scale=w.scale)
            done = hi
        rates.append(done / (time.perf_counter() - t0))
        if done < w.T or time.perf_counter() - t_all > budget_s:
            break
    el = time.perf_counter() - t_all
    return {"value": float(np.median(rates)), "unit": "tokens/s", "cores": blas_threads(),
            "kind": "oracle", **host_cpu(),
            "sample": f"fp64 numpy oracle forward+backward over tokens [0, {done}) of the same stream "
                      f"in {chunk}-token slices with their window halo; median of {len(rates)} "
                      f"pass(es), {el:.1f} s in all"}


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


def copy_bandwidth(mib: int = 1024, reps: int = 10) -> dict:
    """Achievable HBM bandwidth of a plain device copy (read + write) of `mib`
    MiB on this GPU, median of `reps` copies timed with events: the practical
    ceiling beside the 8 TB/s peak.  Run after the timed steps."""
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    evs = [(TimingEvent(), TimingEvent()) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)[reps // 2]
    moved = 2 * (mib << 20)
    del src, dst
    return {"GBps": round(moved / (ms * 1e-3) / 1e9, 1), "bytes_per_copy": moved,
            "frac_of_peak": round(moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}


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
    done = 0
    t0 = time.perf_counter()
    while done < w.T and time.perf_counter() - t0 < budget_s:
        lo, hi = done, min(w.T, done + chunk)
        xs = [x[lo:hi] for x in w.xs]
        mo.forward(xs, w.a[lo:hi])
        mo.backward(xs, w.a[lo:hi], [d[lo:hi] for d in w.dys])
        done = hi
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            **host_cpu(),
            "sample": f"fp64 oracle forward+backward over tokens [0, {done}) of the same stream, "
                      f"in {chunk}-token slices; {el:.1f} s"}


DCMHA_METRIC = "DCMHA composition attention fwd+bwd tokens/s on 1 MI355X (GPT-2-small shape)"
DCMHA_KERNELS = ("dcmha_fwd", "dcmha_bwd_q", "dcmha_bwd_kv")
DCMHA_PASSES = {"dcmha_fwd": ("dcmha_fwd",), "dcmha_bwd": ("dcmha_bwd_q", "dcmha_bwd_kv")}
DCMHA_SOURCES = ("ldc_device.hpp", "ldc_pipeline.hpp", "dcmha.hip", "dcmha_internal.h")


def dcmha_spec_bytes_per_token(H: int, d: int, elem: int) -> dict:
    """Compulsory HBM bytes per token of each DCMHA pass (every tensor of the
    definition once, O in the storage dtype): forward Q, K, V, CS, CW, doc in,
    O out; backward Q, K, V, dO, CS, CW, doc in, dQ, dK, dV (float32), dCS,
    dCW out."""
    row, comp = H * d, 4 * H * H
    return {"dcmha_fwd": 3 * row * elem + 2 * comp + 4 + row * elem,
            "dcmha_bwd": 4 * row * elem + 2 * comp + 4 + 3 * row * 4 + 2 * comp}


def dcmha_design_bytes_per_token(H: int, d: int, elem: int) -> dict:
    """Bytes per token each DCMHA kernel moves as designed: its operands once,
    float32 O and gradients, and the per-head bands the kernels hand each
    other (512 B per token and head each): P and R saved by the forward, P
    read by bwd_q, dS written by bwd_q and read by bwd_kv with R."""
    row, comp, band = H * d, 4 * H * H, 512 * H
    return {
        "dcmha_fwd": 3 * row * elem + 2 * comp + 4 + row * 4 + 2 * band,
        "dcmha_bwd_q": 4 * row * elem + 2 * comp + 4 + band + row * 4 + 2 * comp + band,
        "dcmha_bwd_kv": 2 * row * elem + 4 + 2 * band + 2 * row * 4,
    }


def dcmha_cpu_baseline(w, budget_s: float, chunk: int = 256):
    """Time the fp64 DCMHA oracle (forward + backward) on leading slices of
    the stream (each with its window halo) until `budget_s` seconds."""
    from oracle import dcmha_oracle as dco
    done = 0
    t0 = time.perf_counter()
    while done < w.T and time.perf_counter() - t0 < budget_s:
        lo, hi = done, min(w.T, done + chunk)
        a0 = max(0, lo - w.window + 1)
        sl = lambda x: x[a0:hi]
        qs = range(lo - a0, hi - a0)
        dco.forward(sl(w.q), sl(w.k), sl(w.v), sl(w.cs), sl(w.cw), sl(w.doc), window=w.window,
                    scale=w.scale, queries=qs)
        dco.backward(sl(w.q), sl(w.k), sl(w.v), sl(w.cs), sl(w.cw), sl(w.doc), sl(w.do),
                     window=w.window, scale=w.scale)
        done = hi
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            **host_cpu(),
            "sample": f"fp64 DCMHA oracle forward (the slice's queries) + backward (the slice with its "
                      f"{w.window - 1}-token halo) over tokens [0, {done}) of the same stream in "
                      f"{chunk}-token slices; {el:.1f} s"}


def bench_dcmha(args):
    import torch
    import dynamic_head_composition_amd as ldc
    from dynamic_head_composition_amd import dcmha
    from dynamic_head_composition_amd import workloads as wl

    ldc.load_library()  # fails loudly when the HIP library is missing
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    cfg = dict(wl.DCMHA_BENCH)
    if args.tokens:
        cfg["T"] = args.tokens
        cfg["name"] += f"_trunc{args.tokens}"
    log(f"generating DCMHA workload {cfg} ...")
    w = wl.make_dcmha_workload(**cfg)
    x = w.torch_inputs("cuda")
    T, H, d = w.T, w.H, w.d
    elem = 2 if w.dtype == "bf16" else 4
    code = ldc.LDC_BF16 if w.dtype == "bf16" else ldc.LDC_F32
    f32 = dict(dtype=torch.float32, device="cuda")
    o = torch.empty((T, H, d), **f32)
    grads = tuple(torch.empty(s, **f32) for s in ((T, H, d),) * 3 + ((T, H, H),) * 2)
    ws = torch.empty(max(16, dcmha.workspace_bytes(code, T, H, d, w.window)), dtype=torch.uint8, device="cuda")
    saved = torch.empty(max(16, dcmha.saved_bytes(code, T, H, d, w.window)), dtype=torch.uint8, device="cuda")
    ins = (x["q"], x["k"], x["v"], x["cs"], x["cw"], x["doc"])

    def step(evs=None):
        if evs:
            evs[0].record()
        dcmha.fwd(*ins, window=w.window, scale=w.scale, out=o, saved=saved)
        if evs:
            evs[1].record()
        dcmha.bwd(*ins, saved, x["do"], window=w.window, scale=w.scale, out=grads, workspace=ws, part="q")
        if evs:
            evs[2].record()
        dcmha.bwd(*ins, saved, x["do"], window=w.window, scale=w.scale, out=grads, workspace=ws, part="kv")
        if evs:
            evs[3].record()

    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[TimingEvent() for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if not all(bool(torch.isfinite(t).all()) for t in (o,) + grads):
        raise SystemExit("non-finite outputs")
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    span = lambda a_, b_: [evs[i][a_].elapsed_time(evs[i][b_]) for i in range(args.steps)]
    kstat = {kn: stats_us(span(j, j + 1)) for j, kn in enumerate(DCMHA_KERNELS)}
    pstat = {"dcmha_fwd": stats_us(span(0, 1)), "dcmha_bwd": stats_us(span(1, 3))}
    spec = dcmha_spec_bytes_per_token(H, d, elem)
    design = dcmha_design_bytes_per_token(H, d, elem)
    passes = {}
    for pn, kernels in DCMHA_PASSES.items():
        sec = pstat[pn]["median_us"] * 1e-6
        alg = spec[pn] * T
        traffic = measured_traffic(kernels, w.name, DCMHA_SOURCES)
        passes[pn] = {**pstat[pn], "kernels": list(kernels), "alg_bytes_per_launch": alg,
                      "alg_GBps": round(alg / sec / 1e9, 1), "frac": round(alg / sec / 1e9 / HBM_PEAK_GBPS, 4),
                      "design_bytes_per_launch": sum(design[kn] for kn in kernels) * T,
                      "traffic": traffic,
                      "traffic_over_alg": None if traffic is None else round(traffic / alg, 3)}
    per_kernel = {kn: {**kstat[kn], "design_bytes_per_launch": design[kn] * T,
                       "design_GBps": round(design[kn] * T / (kstat[kn]["median_us"] * 1e-6) / 1e9, 1)}
                  for kn in DCMHA_KERNELS}
    dominant = max(DCMHA_PASSES, key=lambda pn: pstat[pn]["median_us"])
    dom = passes[dominant]
    pairs = valid_pairs(w.doc, w.window)
    # MFMA work per admitted pair: forward scores + values 4Hd; backward dR,
    # scores, dQ, dV, dK 10Hd (the H x H compositions are VALU work)
    alg_tflops = 14.0 * H * d * pairs / (ms_per_step * 1e-3) / 1e12
    value = T / (ms_per_step * 1e-3)
    ceiling_tps = HBM_PEAK_GBPS * 1e9 / sum(spec.values())
    line = {
        "metric": DCMHA_METRIC,
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
        "roofline": {"bound": "hbm", "kernel": dominant, "launches": dom["kernels"],
                     "achieved": dom["alg_GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": dom["frac"], "traffic": dom["traffic"],
                     "traffic_over_alg": dom["traffic_over_alg"],
                     "alg_bytes_per_launch": dom["alg_bytes_per_launch"],
                     "design_bytes_per_launch": dom["design_bytes_per_launch"]},
        "mfma_peak_frac": round(alg_tflops / MFMA_BF16_PEAK_TFLOPS, 5),
        "alg_TFLOPs": round(alg_tflops, 2),
        "step_hbm_ceiling_tokens_per_s": round(ceiling_tps, 1),
        "step_roofline_frac": round(value / ceiling_tps, 4),
        "passes": passes,
        "kernels": per_kernel,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        line["cpu_baseline"] = dcmha_cpu_baseline(w, args.cpu_budget)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


FUSED_METRIC = "attention block fwd tokens/s on 1 MI355X (GPT-2-small shape): main attention + LDC fused"
FUSED_SOURCES = ("ldc_device.hpp", "ldc_pipeline.hpp", "ldc_fwd.hip", "ldc_internal.h", "fused.hip",
                 "fused_internal.h")
FUSED_TILE = 128   # queries per work item of the main attention kernel
FUSED_STAGE = 64   # keys per stage


def fused_design_bytes(doc: np.ndarray, H: int, d: int, elem: int) -> int:
    """Bytes the fused call moves as designed, with no reuse between work
    items: the Lightweight DC score pass (Q, K, C, G, doc in; the band and the
    statistics out), the run starts and the item order (doc in, one int per
    token out), and per (128-query tile, head) item its Q rows, every 64-key
    stage of K and V from the tile's earliest run start to its last query,
    the window's 256 V rows staged again for the band's value contraction,
    its G, run starts and band blocks, and its float32 O rows.  Rows that
    neighbouring items share come from the L2, so measured HBM traffic lies
    between the algorithmic bytes and this figure."""
    T = len(doc)
    row = H * d
    starts = np.ones(T, dtype=bool)
    starts[1:] = doc[1:] != doc[:-1]
    rs = np.maximum.accumulate(np.where(starts, np.arange(T), 0))
    q0 = np.arange(0, T, FUSED_TILE)
    span = (q0 - 2 * FUSED_STAGE) - rs[q0]
    stages = np.where(span > 0, (span + FUSED_STAGE - 1) // FUSED_STAGE, 0) + 4
    score_pass = T * (2 * row * elem + 8 * H + 4 + 512 + 8 * H)
    run_starts = T * 12
    per_head_rows = (int(stages.sum()) * 2 * FUSED_STAGE + len(q0) * 256) * d * elem  # K and V stages, restage
    attention = H * per_head_rows + T * (row * elem + 4 * H + 4 * H + 512 * H + row * 4)
    return int(score_pass + run_starts + attention)


def fused_cpu_baseline(w, budget_s: float, chunk: int = 512):
    """Time the fp64 fused-block oracle on leading query slices of the stream
    (each query with its whole run and window) until `budget_s` seconds."""
    from oracle import fused_oracle as fo
    from oracle import ldc_oracle as orc
    done = 0
    t0 = time.perf_counter()
    while done < w.T and time.perf_counter() - t0 < budget_s:
        lo, hi = done, min(w.T, done + chunk)
        fo.main_attention(w.q, w.k, w.v, w.doc, w.scale, queries=range(lo, hi))
        orc.forward_slice(w.q, w.k, w.v, w.c, w.g, w.doc, lo, hi, window=w.window, scale=w.scale)
        done = hi
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            **host_cpu(),
            "sample": f"fp64 oracle of the block (main attention of each query over its run + the "
                      f"Lightweight DC layer) over queries [0, {done}) of the same stream in "
                      f"{chunk}-query slices; {el:.1f} s"}


def bench_fused(args):
    """The block's attention forward with the Lightweight DC layer fused into
    the main attention kernel; the unfused pair (main attention alone, then the
    Lightweight DC forward) timed beside it."""
    import torch
    import dynamic_head_composition_amd as ldc
    from dynamic_head_composition_amd import fused
    from dynamic_head_composition_amd import workloads as wl

    ldc.load_library()  # fails loudly when the HIP library is missing
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    log("generating workload 1 ...")
    w = wl.config_workload(1, T=args.tokens)
    if args.window:
        w.window = args.window
        w.name += f"_win{args.window}"
    x = w.torch_inputs("cuda", with_do=False)
    T, H, d = w.T, w.H, w.d
    elem = 2 if w.dtype == "bf16" else 4
    f32 = dict(dtype=torch.float32, device="cuda")
    o, m, lo_ = (torch.empty((T, H, d), **f32) for _ in range(3))
    ins = (x["q"], x["k"], x["v"], x["c"], x["g"], x["doc"])
    code = ldc.LDC_BF16 if w.dtype == "bf16" else ldc.LDC_F32
    ws = torch.empty(max(16, fused.workspace_bytes(code, T, H, d, w.window)), dtype=torch.uint8, device="cuda")
    ws_m = torch.empty(max(16, fused.main_workspace_bytes(T)), dtype=torch.uint8, device="cuda")

    def step():
        fused.fwd(*ins, window=w.window, scale=w.scale, out=o, workspace=ws)

    def unfused(evs):
        evs[0].record()
        fused.main_fwd(x["q"], x["k"], x["v"], x["doc"], scale=w.scale, out=m, workspace=ws_m)
        evs[1].record()
        ldc.fwd(*ins, window=w.window, scale=w.scale, out=lo_)
        evs[2].record()

    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[TimingEvent() for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record()
        step()
        evs[i][1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if not bool(torch.isfinite(o).all()):
        raise SystemExit("non-finite outputs")
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    fst = stats_us([e[0].elapsed_time(e[1]) for e in evs])
    # the unfused pair, for comparison (not part of the step)
    uevs = [[TimingEvent() for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        unfused(uevs[i])
    torch.cuda.synchronize()
    mst = stats_us([e[0].elapsed_time(e[1]) for e in uevs])
    lst = stats_us([e[1].elapsed_time(e[2]) for e in uevs])
    ust = stats_us([e[0].elapsed_time(e[2]) for e in uevs])

    main_pairs = valid_pairs(w.doc, T)          # every key of the query's run up to the query
    ldc_pairs = valid_pairs(w.doc, w.window)
    # MFMA work per admitted pair and head: the score (2d) and the value
    # contraction (2d), for the main attention and the Lightweight DC branch
    flops = 4.0 * H * d * (main_pairs + ldc_pairs)
    sec = fst["median_us"] * 1e-6
    achieved = flops / sec / 1e12
    alg_bytes = spec_bytes_per_token(H, d, elem)["ldc_fwd"] * T  # Q, K, V, C, G, doc in; O out
    value = T / (ms_per_step * 1e-3)
    line = {
        "metric": FUSED_METRIC,
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
                   "recipe": w.recipe, "main_pairs": main_pairs, "ldc_pairs": ldc_pairs,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "fused_fwd", "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(("fused_fwd",), w.name, FUSED_SOURCES),
                     "alg_flops_per_launch": flops, "alg_bytes_per_launch": alg_bytes,
                     "design_bytes_per_launch": fused_design_bytes(w.doc, H, d, elem),
                     "hbm_frac": round(alg_bytes / sec / 1e9 / HBM_PEAK_GBPS, 4)},
        "kernels": {"fused_fwd": fst, "main_attention_fwd": mst, "ldc_fwd": lst},
        "unfused_us": ust,
        "fused_speedup_vs_unfused": round(ust["median_us"] / fst["median_us"], 3),
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        line["cpu_baseline"] = fused_cpu_baseline(w, args.cpu_budget)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


CG_METRIC = "C/G generator fwd+bwd tokens/s on 1 MI355X (GPT-2-small hidden state)"
CG_KERNELS = ("cg_fwd", "cg_bwd")
CG_SOURCES = ("ldc_device.hpp", "cg.hip", "cg_internal.h")


def cg_bytes_per_token(dm: int, H: int, elem: int) -> dict:
    """Compulsory HBM bytes per token of the generator's passes: forward x in,
    C and G out; backward x, dC, dG in, dx (float32) out (the weights and
    their gradients are a few KB per launch)."""
    return {"cg_fwd": dm * elem + 8 * H, "cg_bwd": dm * elem + 8 * H + dm * 4}


def bench_cg(args):
    import torch
    import dynamic_head_composition_amd as ldc
    from dynamic_head_composition_amd import cg
    from dynamic_head_composition_amd import workloads as wl

    ldc.load_library()  # fails loudly when the HIP library is missing
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    cfg = dict(wl.CG_BENCH)
    if args.tokens:
        cfg["T"] = args.tokens
        cfg["name"] += f"_trunc{args.tokens}"
    log(f"generating generator workload {cfg} ...")
    w = wl.make_cg_workload(**cfg)
    x = w.torch_inputs("cuda")
    T, dm, H = w.T, w.dm, w.H
    elem = 2 if w.dtype == "bf16" else 4
    f32 = dict(dtype=torch.float32, device="cuda")
    cgo = (torch.empty((T, H), **f32), torch.empty((T, H), **f32))
    grads = (torch.empty((T, dm), **f32), torch.empty((dm, H), **f32), torch.empty((dm, H), **f32))
    ws = torch.empty(max(16, cg.workspace_bytes(0 if w.dtype == "bf16" else 1, T, dm, H)), dtype=torch.uint8,
                     device="cuda")

    def step(evs=None):
        if evs:
            evs[0].record()
        cg.fwd(x["x"], x["wc"], x["wg"], out=cgo)
        if evs:
            evs[1].record()
        cg.bwd(x["x"], x["wc"], x["wg"], x["dc"], x["dg"], out=grads, workspace=ws)
        if evs:
            evs[2].record()

    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[TimingEvent() for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if not all(bool(torch.isfinite(t).all()) for t in cgo + grads):
        raise SystemExit("non-finite outputs")
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kstat = {kn: stats_us([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)])
             for j, kn in enumerate(CG_KERNELS)}
    bpt = cg_bytes_per_token(dm, H, elem)
    per_kernel = {kn: {**kstat[kn], "alg_bytes_per_launch": bpt[kn] * T,
                       "alg_GBps": round(bpt[kn] * T / (kstat[kn]["median_us"] * 1e-6) / 1e9, 1)}
                  for kn in CG_KERNELS}
    dominant = max(CG_KERNELS, key=lambda kn: kstat[kn]["median_us"])
    achieved = per_kernel[dominant]["alg_GBps"]
    value = T / (ms_per_step * 1e-3)
    ceiling_tps = HBM_PEAK_GBPS * 1e9 / sum(bpt.values())
    line = {
        "metric": CG_METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": T, "model_dim": dm, "heads": H, "recipe": w.recipe,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic([dominant], w.name, CG_SOURCES),
                     "alg_bytes_per_launch": bpt[dominant] * T},
        "step_hbm_ceiling_tokens_per_s": round(ceiling_tps, 1),
        "step_roofline_frac": round(value / ceiling_tps, 4),
        "kernels": per_kernel,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        from oracle import cg_oracle as cgor
        done, t_0, chunk = 0, time.perf_counter(), 4096
        while done < T and time.perf_counter() - t_0 < args.cpu_budget:
            lo, hi = done, min(T, done + chunk)
            cgor.forward(w.x[lo:hi], w.wc, w.wg)
            cgor.backward(w.x[lo:hi], w.wc, w.wg, w.dc[lo:hi], w.dg[lo:hi])
            done = hi
        el = time.perf_counter() - t_0
        line["cpu_baseline"] = {"value": done / el, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
                                **host_cpu(),
                                "sample": f"fp64 oracle forward+backward over tokens [0, {done}) in {chunk}-token "
                                          f"slices (dW summed per slice); {el:.1f} s"}
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


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
    evs = [[TimingEvent() for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if not all(bool(torch.isfinite(t).all()) for t in ys + dxs + [da]):
        raise SystemExit("non-finite outputs")
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kstat = {kn: stats_us([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)])
             for j, kn in enumerate(MUDD_KERNELS)}
    bpt = mudd_bytes_per_token(dm, W, J, elem)
    per_kernel = {kn: {**kstat[kn], "alg_bytes_per_launch": bpt[kn] * T,
                       "alg_GBps": round(bpt[kn] * T / (kstat[kn]["median_us"] * 1e-6) / 1e9, 1)}
                  for kn in MUDD_KERNELS}
    dominant = max(MUDD_KERNELS, key=lambda kn: kstat[kn]["median_us"])
    achieved = bpt[dominant] * T / (kstat[dominant]["median_us"] * 1e-6) / 1e9
    traffic = measured_traffic([dominant], w.name, MUDD_SOURCES)
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
                     "traffic": traffic,
                     "traffic_over_alg": None if traffic is None else round(traffic / (bpt[dominant] * T), 3)},
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
    ap.add_argument("--workload", choices=("ldc", "dcmha", "cg", "mudd", "fused"), default="ldc",
                    help="ldc: the Lightweight DC layer (default); dcmha: full DCMHA composition at "
                         "the same shape; cg: the generator of C and G from the hidden state; "
                         "mudd: MUDD layer mixing; fused: the block's main attention with the "
                         "Lightweight DC layer fused in (forward)")
    ap.add_argument("--tokens", type=int, default=None, help="truncate the stream (quick runs only)")
    ap.add_argument("--window", type=int, default=None,
                    help="another Lightweight DC window (1-128) on the same stream, for the ldc and "
                         "fused workloads (not the headline configuration)")
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
    if args.workload == "dcmha":
        return bench_dcmha(args)
    if args.workload == "cg":
        return bench_cg(args)
    if args.workload == "fused":
        return bench_fused(args)

    import torch
    import dynamic_head_composition_amd as ldc
    from dynamic_head_composition_amd import workloads as wl

    ldc.load_library()  # fails loudly when the HIP library is missing
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")

    log(f"generating workload {args.config} ...")
    w = wl.config_workload(args.config, T=args.tokens)
    if args.window:
        w.window = args.window
        w.name += f"_win{args.window}"
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
    evs = [[TimingEvent() for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if not all(bool(torch.isfinite(t).all()) for t in (o,) + grads):
        raise SystemExit("non-finite outputs")

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    span = lambda a, b: [evs[i][a].elapsed_time(evs[i][b]) for i in range(args.steps)]
    # events: 0 before ldc_fwd, 1 after it, 2 after ldc_bwd_q, 3 after ldc_bwd_kv
    kstat = {kn: stats_us(span(j, j + 1)) for j, kn in enumerate(KERNELS)}
    pstat = {"ldc_fwd": stats_us(span(0, 1)), "ldc_bwd": stats_us(span(1, 3))}
    pairs = valid_pairs(w.doc, w.window)
    total_flops = 14.0 * H * d * pairs
    spec = spec_bytes_per_token(H, d, elem)
    design = design_bytes_per_token(H, d, elem)
    passes = {}
    for pn, kernels in PASSES.items():
        sec = pstat[pn]["median_us"] * 1e-6
        alg = spec[pn] * T
        traffic = measured_traffic(kernels, w.name)
        passes[pn] = {**pstat[pn], "kernels": list(kernels), "alg_bytes_per_launch": alg,
                      "alg_GBps": round(alg / sec / 1e9, 1),
                      "frac": round(alg / sec / 1e9 / HBM_PEAK_GBPS, 4),
                      "design_bytes_per_launch": sum(design[kn] for kn in kernels) * T,
                      "traffic": traffic,
                      "traffic_over_alg": None if traffic is None else round(traffic / alg, 3)}
    per_kernel = {kn: {**kstat[kn], "design_bytes_per_launch": design[kn] * T} for kn in KERNELS}
    dominant = max(PASSES, key=lambda pn: pstat[pn]["median_us"])
    dom = passes[dominant]
    value = T / (ms_per_step * 1e-3)
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    alg_tflops = total_flops / (ms_per_step * 1e-3) / 1e12
    ceiling_tps = HBM_PEAK_GBPS * 1e9 / sum(spec.values())

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
        "roofline": {"bound": "hbm", "kernel": dominant, "launches": dom["kernels"],
                     "achieved": dom["alg_GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": dom["frac"], "traffic": dom["traffic"],
                     "traffic_over_alg": dom["traffic_over_alg"],
                     "alg_bytes_per_launch": dom["alg_bytes_per_launch"],
                     "design_bytes_per_launch": dom["design_bytes_per_launch"]},
        "mfma_peak_frac": round(alg_tflops / mfma_peak, 5),
        "alg_TFLOPs": round(alg_tflops, 2),
        "step_hbm_ceiling_tokens_per_s": round(ceiling_tps, 1),
        "step_roofline_frac": round(value / ceiling_tps, 4),
        "passes": passes,
        "kernels": per_kernel,
    }
    # after the timed steps: the achievable HBM rate of a plain copy on this GPU
    line["hbm_copy_probe"] = copy_bandwidth()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
