"""The benchmark's output contract on a real run (a short one, in a child
process): one JSON line with the fields the driver reads, a roofline object
for the slower kernel, and per-kernel durations consistent with the
event-timed step."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "20", "--warmup", "2",
                        "--no-cpu-baseline", "--no-copy-ceiling", *args],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.strip().splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def test_default_workload_line():
    d = run_bench()
    for key, want in (("n_gpus", 1), ("steps", 20), ("warmup", 2), ("higher_is_better", True),
                      ("scaling", "weak"), ("vs_baseline", None), ("data", "synthetic"), ("unit", "GB/s")):
        assert d[key] == want, key
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["gpu_ms_per_step"] > 0
    assert d["config"]["workload"] == "moe_bwd_jagged"
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0 and roof["unit"] == "GB/s"
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert roof["traffic"] is None or roof["traffic"] > roof["algorithmic_bytes_per_launch"] * 0.9
    kernels = d["kernels"]
    assert len(kernels) == 2
    slower = max(kernels.values(), key=lambda k: k["avg_us"])
    assert roof["avg_launch_us"] == slower["avg_us"]
    for k in kernels.values():
        assert 0 < k["avg_us"] <= k["interval_avg_us"]
        assert abs(k["GBps"] - k["algorithmic_bytes"] / (k["avg_us"] * 1e-6) / 1e9) < 1.0
    # the kernels' durations add up to the event-timed step (launch gaps aside)
    total_us = sum(k["avg_us"] for k in kernels.values())
    assert abs(total_us - d["gpu_ms_per_step"] * 1e3) < 0.1 * total_us


def test_cold_timings_and_single_kernel_workload():
    d = run_bench("--workload", "blockwise", "--flush-iters", "5")
    for k in d["kernels"].values():
        assert k["flushed_us"]["iters"] == 5
        assert k["flushed_us"]["min"] <= k["flushed_us"]["median"] <= k["flushed_us"]["max"]
    assert d["config"]["workload"] == "blockwise"
