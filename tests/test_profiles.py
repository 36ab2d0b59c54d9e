"""Consistency of the committed rocprofv3 traffic record with the code (CPU).

Workloads: the Lightweight DC configurations, the DCMHA composition, the C/G
generator and MUDD mixing, each with the kernel sources its entries were
taken on.

profiles/hbm_traffic.json holds measured HBM bytes per launch, tagged with a
digest of the kernel sources they were taken on; bench.py reports them only
while the digest matches.  For every pass of the layer whose launches all have
a matching entry, the test reports the measured traffic over the algorithmic
bytes of the pass (the compulsory I/O of the definition, bench.spec_bytes_per_
token) and checks that it is at least the algorithmic bytes and equals the
ratio the record states.  Each entry must also sit within 10% above the bytes
its kernel moves as designed (nothing re-read from HBM beyond halo rows), and
the summary it names must exist and carry the commands that produced it."""
import json
import os

import pytest

import bench
from dynamic_head_composition_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REC = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def ldc_config(workload: str) -> dict:
    return next(v for v in wl.CONFIGS.values() if v["name"] == workload)


def design(workload: str) -> dict:
    if workload.startswith("mudd_"):
        c = wl.MUDD_BENCH
        bpt = bench.mudd_bytes_per_token(c["dm"], c["W"], c["J"], 2 if c["dtype"] == "bf16" else 4)
        return {k: v * c["T"] for k, v in bpt.items()}
    if workload.startswith("dcmha_"):
        c = wl.DCMHA_BENCH
        bpt = bench.dcmha_design_bytes_per_token(c["H"], c["d"], 2 if c["dtype"] == "bf16" else 4)
        return {k: v * c["T"] for k, v in bpt.items()}
    if workload.startswith("cg_"):
        c = wl.CG_BENCH
        bpt = bench.cg_bytes_per_token(c["dm"], c["H"], 2 if c["dtype"] == "bf16" else 4)
        return {k: v * c["T"] for k, v in bpt.items()}
    cfg = ldc_config(workload)
    bpt = bench.design_bytes_per_token(cfg["H"], cfg["d"], 2 if cfg["dtype"] == "bf16" else 4)
    return {k: v * cfg["T"] for k, v in bpt.items()}


def entries():
    rec = json.load(open(REC))
    for workload, kernels in rec.items():
        for kernel, ent in kernels.items():
            if kernel.startswith("_"):
                continue
            yield workload, kernel, ent


def sources(kernel):
    if kernel == "fused_fwd":
        return bench.FUSED_SOURCES
    if kernel.startswith("mudd_"):
        return bench.MUDD_SOURCES
    if kernel.startswith("dcmha_"):
        return bench.DCMHA_SOURCES
    if kernel.startswith("cg_"):
        return bench.CG_SOURCES
    return bench.SOURCES


@pytest.mark.parametrize("workload,kernel,ent", list(entries()), ids=lambda x: x if isinstance(x, str) else "")
def test_traffic_record(workload, kernel, ent):
    summary = os.path.join(ROOT, "profiles", ent["summary"])
    text = open(summary).read()
    assert "rocprofv3 --kernel-trace --stats" in text and "--pmc FETCH_SIZE" in text and "--pmc WRITE_SIZE" in text
    assert abs(ent["read_bytes"] + ent["write_bytes"] - ent["bytes_per_launch"]) <= 2  # each rounded down
    if ent["source_digest"] != bench.source_digest(sources(kernel)):
        pytest.skip("kernel sources changed since the counters were taken (bench reports traffic null)")
    if kernel == "fused_fwd":
        # the main attention re-stages each document's earlier K and V rows
        # per query tile, so the traffic lies between the block's algorithmic
        # bytes and its design bytes with no reuse between work items
        cfg = ldc_config(workload)
        w = wl.config_workload(next(i for i, v in wl.CONFIGS.items() if v["name"] == workload))
        elem = 2 if cfg["dtype"] == "bf16" else 4
        alg = bench.spec_bytes_per_token(cfg["H"], cfg["d"], elem)["ldc_fwd"] * cfg["T"]
        top = bench.fused_design_bytes(w.doc, cfg["H"], cfg["d"], elem)
        assert alg <= ent["bytes_per_launch"] <= top, (ent["bytes_per_launch"], alg, top)
        return
    alg = design(workload)[kernel]
    assert 0.98 * alg <= ent["bytes_per_launch"] <= 1.10 * alg, (ent["bytes_per_launch"], alg)


def pass_cases():
    rec = json.load(open(REC))
    for workload in rec:
        if workload.startswith(("mudd_", "dcmha_", "cg_")) or "fused_fwd" in rec[workload]:
            continue
        for pn in bench.PASSES:
            yield workload, pn


@pytest.mark.parametrize("workload,pn", list(pass_cases()))
def test_pass_traffic_over_algorithmic(workload, pn):
    """Measured traffic of a pass against the definition's compulsory bytes."""
    cfg = ldc_config(workload)
    traffic = bench.measured_traffic(bench.PASSES[pn], workload)
    if traffic is None:
        pytest.skip("no record taken on the current kernel sources")
    spec = bench.spec_bytes_per_token(cfg["H"], cfg["d"], 2 if cfg["dtype"] == "bf16" else 4)[pn] * cfg["T"]
    ratio = traffic / spec
    print(f"{workload} {pn}: traffic {traffic / 1e6:.1f} MB / algorithmic {spec / 1e6:.1f} MB = {ratio:.3f}")
    assert ratio >= 0.98
    stated = json.load(open(REC))[workload].get("_passes", {}).get(pn)
    if stated is not None:
        assert abs(stated["traffic_over_alg"] - ratio) < 5e-3, (stated, ratio)


def test_current_kernels_have_a_matching_record():
    rec = json.load(open(REC))
    ldc = rec["gpt2s_fwdbwd_T65536_H6_d128"]["ldc_fwd"]["source_digest"]
    mudd = rec["mudd_T65536_dm768_W4_J13_bf16"]["mudd_bwd"]["source_digest"]
    assert mudd == bench.source_digest(bench.MUDD_SOURCES)
    if ldc != bench.source_digest(bench.SOURCES):
        pytest.skip("LDC kernel sources changed since the counters were taken (bench reports traffic null)")
