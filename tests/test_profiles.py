"""Consistency of the committed rocprofv3 traffic record with the code (CPU).

profiles/hbm_traffic.json holds measured HBM bytes per launch, tagged with a
digest of the kernel sources they were taken on; bench.py reports them only
while the digest matches.  For every matching entry the measured traffic must
sit close above the algorithmic bytes bench.py computes (nothing re-read from
HBM beyond the halo rows), and the summary it names must exist and carry the
commands that produced it."""
import json
import os

import pytest

import bench
from dynamic_head_composition_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REC = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def algorithmic(workload: str) -> dict:
    if workload.startswith("mudd_"):
        c = wl.MUDD_BENCH
        bpt = bench.mudd_bytes_per_token(c["dm"], c["W"], c["J"], 2 if c["dtype"] == "bf16" else 4)
        return {k: v * c["T"] for k, v in bpt.items()}
    cfg = next(v for v in wl.CONFIGS.values() if v["name"] == workload)
    bpt = bench.algorithmic_bytes_per_token(cfg["H"], cfg["d"], 2 if cfg["dtype"] == "bf16" else 4)
    return {k: v * cfg["T"] for k, v in bpt.items()}


def entries():
    rec = json.load(open(REC))
    for workload, kernels in rec.items():
        for kernel, ent in kernels.items():
            yield workload, kernel, ent


@pytest.mark.parametrize("workload,kernel,ent", list(entries()), ids=lambda x: x if isinstance(x, str) else "")
def test_traffic_record(workload, kernel, ent):
    files = bench.MUDD_SOURCES if kernel.startswith("mudd_") else bench.SOURCES
    summary = os.path.join(ROOT, "profiles", ent["summary"])
    text = open(summary).read()
    assert "rocprofv3 --kernel-trace --stats" in text and "--pmc FETCH_SIZE" in text and "--pmc WRITE_SIZE" in text
    assert abs(ent["read_bytes"] + ent["write_bytes"] - ent["bytes_per_launch"]) <= 2  # each rounded down
    if ent["source_digest"] != bench.source_digest(files):
        pytest.skip("kernel sources changed since the counters were taken (bench reports traffic null)")
    alg = algorithmic(workload)[kernel]
    assert 0.98 * alg <= ent["bytes_per_launch"] <= 1.10 * alg, (ent["bytes_per_launch"], alg)


def test_current_kernels_have_a_matching_record():
    rec = json.load(open(REC))
    ldc = rec["gpt2s_fwdbwd_T65536_H6_d128"]["ldc_bwd_kv"]["source_digest"]
    mudd = rec["mudd_T65536_dm768_W4_J13_bf16"]["mudd_bwd"]["source_digest"]
    assert ldc == bench.source_digest(bench.SOURCES)
    assert mudd == bench.source_digest(bench.MUDD_SOURCES)
