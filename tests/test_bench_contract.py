"""The bench's command-line contract: one JSON line with the headline metric,
the roofline of the dominant kernel and (unless skipped) the oracle baseline;
more than one GPU is refused with a message."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    # the check runs before anything touches a GPU
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


@pytest.mark.gpu
def test_bench_json_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "2",
                        "--no-cpu-baseline", "--no-decode", "--no-backward", "--no-projection", "--no-variants",
                        "--no-diagnostic", "--no-others", "--settle", "0.05", "--blocks", "3"], capture_output=True, text=True,
                       timeout=280, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ["metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline"]:
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"] == "dense_prefill"
    rf = d["roofline"]
    for k in ["bound", "achieved", "peak", "unit", "frac", "traffic"]:
        assert k in rf, k
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    # achieved follows from the event-timed average launch duration of the forward
    assert abs(rf["achieved"] - rf["algorithmic_flops_per_launch"] / (rf["avg_launch_ms"] * 1e-3) / 1e12) < 1e-6
    t = d["timing"]
    assert t["min_ms"] <= t["median_ms"] and t["clock_settle_s"] >= 0 and t["blocks"] >= 1
    assert set(d["workloads"]) == {"dense_prefill"}
    assert d["workloads"]["dense_prefill"]["value"] == d["value"]
