"""bench.py's output contract: one JSON line with the fields that benchmark
harnesses and the roofline report read.  The multi-GPU refusal runs on the host; one short
run of the tiny workload runs on the GPU."""

import json
import os
import subprocess
import sys

import pytest

from tests.conftest import ROOT

BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused_with_a_message():
    run = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert run.returncode != 0
    assert "one GPU" in run.stderr


@pytest.mark.gpu
def test_bench_json_line():
    run = subprocess.run([sys.executable, BENCH, "--config", "tiny", "--steps", "5", "--warmup", "5",
                          "--cpu-seconds", "1"], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stderr[-2000:]
    lines = [l for l in run.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 5
    assert d["config"]["workload"] == "tiny"
    assert d["dtype"] == "f32" and d["higher_is_better"] is True
    # value is the step's attention flops over its time (both printed rounded)
    want = d["attention_flops_per_step"] / (d["ms_per_step"] * 1e-3) / 1e12
    assert abs(d["value"] - want) <= 0.01 * want + 0.006
    r = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in r, key
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    rs = d["roofline_share"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic", "R", "flops_per_launch", "avg_launch_ms"):
        assert key in rs, key
    assert rs["R"] == 1 and abs(rs["frac"] - rs["achieved"] / rs["peak"]) < 1e-3
    want_share = rs["flops_per_launch"] / (rs["avg_launch_ms"] * 1e-3) / 1e12
    assert abs(rs["achieved"] - want_share) <= 0.01 * want_share + 0.006
    c = d["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in c, key
    assert c["kind"] == "oracle" and c["timed_output_vs_oracle"]["ok"]
    assert d["checks"]["output_finite"] and d["checks"]["relayout_round_trip_bytes_equal"]
