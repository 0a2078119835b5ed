"""bench.py end to end on the GPU, at a small size: the one JSON line it prints carries the
fields the benchmark contract asks for, with values consistent among themselves (µs per token
against ms per step, the roofline fraction against its achieved and peak rates), and the
oracle's host-core baseline.  Two layers instead of 32, so no recorded traffic figure applies
(the recorded one belongs to the full default workload) and `traffic` must be null."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("workload", ["decode7b", "decode7b-int4"])
def test_bench_json_line(workload):
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", workload,
           "--layers", "2", "--tokens", "2", "--steps", "2", "--warmup", "1", "--cpu-layers", "1",
           "--no-dense", "--no-read-probe", "--no-separate", "--no-deterministic"]
    print("bench:", " ".join(cmd[2:]), flush=True)
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    line = r.stdout.strip().splitlines()[-1]
    j = json.loads(line)

    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in j, k
    assert j["n_gpus"] == 1 and j["steps"] == 2 and j["warmup"] == 1
    assert j["unit"] == "us/token" and j["higher_is_better"] is False
    assert j["vs_baseline"] is None and j["data"] == "synthetic"
    assert j["config"]["workload"].startswith(workload + ":")
    assert j["config"]["layers"] == 2 and "2 layers" in j["config"]["workload"]
    assert j["value"] > 0
    per_tok = j["config"]["tokens_per_step"]
    assert abs(j["value"] - j["ms_per_step"] * 1e3 / per_tok) <= 0.01 * j["value"] + 0.01

    rf = j["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0.0 < rf["frac"] < 1.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["traffic"] is None and rf["traffic_source"] is None
    assert rf["kernel"] == "fused_phase_kernel<%s>" % ("fp16" if workload == "decode7b" else "int4")

    cpu = j["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0
    assert cpu["unit"] == "us/token" and cpu["sample"]

    assert j["batched"] is not None and j["batched"]["value"] > 0


def test_bench_tier_fit():
    """--tier-fit at two layers: three FULL-only and three APPROX-only points per tier, the
    bytes growing with the fraction of channels selected, and a finite line per tier for both
    the layer-serial and the batched form."""
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--layers", "2", "--tokens", "2",
           "--steps", "2", "--warmup", "1", "--tier-fit", "--no-cpu-baseline", "--no-dense",
           "--no-read-probe", "--no-separate", "--no-deterministic"]
    print("bench:", " ".join(cmd[2:]), flush=True)
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    tf = json.loads(r.stdout.strip().splitlines()[-1])["tier_fit"]
    for tier, col in (("FULL", "full"), ("APPROX", "approx")):
        pts = tf[tier]["points"]
        assert len(pts) == 3
        assert all(p[col] > 0 and p["approx" if col == "full" else "full"] == 0 for p in pts)
        mb = [p["MB_per_launch"] for p in pts]
        assert mb == sorted(mb) and mb[0] > 0
        assert all(p["us_per_launch"] > 0 and p["batched_us_per_step"] > 0 for p in pts)
        for form in ("layer_serial", "batched"):
            line = tf[tier][form]
            assert all(isinstance(v, float) and v == v for k, v in line.items()
                       if k != "marginal_TBps"), line
