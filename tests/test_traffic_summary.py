"""The committed rocprofv3 traffic summary: the forward scan moves no more HBM
bytes than its inputs and outputs, and bench.py reports the same figures.

The summary (profiles/traffic__forward_scan__*.md) holds FETCH_SIZE and
WRITE_SIZE per dispatch scaled by the factors a 1 GiB copy gave in the same
run.  The expanded (batch, dim, seqlen, dstate) state would be 16x the y
tensor in fp32: a kernel that stored it, or spilled it through HBM, would
fail the ratios below by an order of magnitude.
"""
import glob
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _summary():
    paths = glob.glob(os.path.join(ROOT, "profiles", "traffic__forward_scan__*.md"))
    assert len(paths) == 1, paths
    text = open(paths[0]).read()
    return json.loads(text.split("```json")[1].split("```")[0])


def test_calibration_factors_are_sane():
    s = _summary()
    # A plain copy reads each byte once and writes it once: the counters may
    # count in other units, but by a fixed small factor.
    assert 0.5 <= s["fetch_factor"] <= 4.0
    assert 0.5 <= s["write_factor"] <= 4.0


@pytest.mark.parametrize("workload", ["Mamba-1.4B layer, bf16", "Mamba-130M layer, fp32", "long sequence, fp32"])
def test_single_pass_traffic_within_bar(workload):
    """Every workload runs one pass over the sequence (the single-pass kernel
    on the layer workloads, the chunked kernel on the long sequence): writes
    within 1.1x and reads + writes within 1.25x of the algorithmic bytes."""
    w = _summary()["workloads"][workload]
    assert w["write_ratio"] <= 1.10, w
    assert w["total_ratio"] <= 1.25, w
    assert w["read_ratio"] >= 0.95 and w["write_ratio"] >= 0.95, w  # the counters saw the whole call


def test_bench_reports_the_measured_figures():
    import sys
    sys.path.insert(0, ROOT)
    import bench
    s = _summary()
    m = bench.MEASURED_TRAFFIC
    assert m["source_sha256"] == s["source_sha256"]
    names = {2: "Mamba-1.4B layer, bf16", 1: "Mamba-130M layer, fp32", 3: "long sequence, fp32"}
    for cfg, name in names.items():
        assert m["per_call"][cfg]["read_bytes"] == s["workloads"][name]["read_bytes"]
        assert m["per_call"][cfg]["write_bytes"] == s["workloads"][name]["write_bytes"]
