"""The benchmark's output contract on real runs (in child processes): one
JSON line with the fields the driver reads, a roofline object from the
dominant kernel's cold (flushed) median, cold and warm per-kernel timings,
extra workloads, the streaming ceiling and the run metadata.

The headline workload's input (5.4 GB) is far larger than the caches, so
the two independent timings of its single kernel — K launches back to back
between one event pair, and single launches after a 1 GiB flush — must
agree closely."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, timeout=600):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "10", "--warmup", "2",
                        "--flush-iters", "5", *args],
                       capture_output=True, text=True, timeout=timeout, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.strip().splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def check_kernel(k):
    c = k["cold_us"]
    assert c["iters"] == 5 and 0 < c["min"] <= c["median"] <= c["max"]
    assert k["warm_us"] > 0
    assert abs(k["GBps_cold"] - k["algorithmic_bytes"] / (c["median"] * 1e-6) / 1e9) < 1.0


@pytest.mark.timeout(900)
def test_default_headline_line():
    d = run_bench("--extras", "blockwise", timeout=850)
    for key, want in (("n_gpus", 1), ("steps", 10), ("warmup", 2), ("higher_is_better", True),
                      ("scaling", "weak"), ("data", "synthetic"), ("unit", "GB/s"),
                      ("dtype", "f32")):
        assert d[key] == want, key
    assert d["config"]["workload"] == "mx3d_E64_sweep"
    # against the pages' own figure for this shape and metric (other hardware)
    assert d["baseline"]["value"] == 4152.11 and d["baseline"]["unit"] == "GB/s"
    assert abs(d["vs_baseline"] - d["value"] / 4152.11) < 1e-3
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["gpu_ms_per_step"] > 0
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0 and roof["unit"] == "GB/s"
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert roof["algorithmic_bytes_per_launch"] == 3 * 64 * 8192 * 5120 + 64 * 256 * 5120
    (k,) = d["kernels"].values()
    check_kernel(k)
    assert roof["avg_launch_us"] == k["cold_us"]["median"]
    # independent timings of the same kernel agree: back-to-back steps
    # (event pair around K launches) against flushed single launches
    step_us = d["gpu_ms_per_step"] * 1e3
    assert abs(step_us - k["cold_us"]["median"]) < 0.05 * step_us
    assert abs(k["warm_us"] - k["cold_us"]["median"]) < 0.05 * step_us
    # the line's value is the step's throughput
    assert abs(d["value"] - roof["algorithmic_bytes_per_launch"] / (d["ms_per_step"] * 1e-3) / 1e9) \
        < 0.01 * d["value"]
    # extras, ceiling, baseline, metadata
    (extra,) = d["workloads"].values()
    assert extra["config"]["workload"] == "blockwise"
    for k in extra["kernels"].values():
        check_kernel(k)
    ceil = d["stream_ceiling"]
    for key in ("read2_write1_GBps", "read2_write1_device_scope_GBps", "read_only_GBps",
                "write_only_GBps", "read1_write1_GBps", "d2d_copy_GBps"):
        assert 500 < ceil[key] < 8000, key
    assert ceil["read2_write1_best_GBps"] == max(ceil["read2_write1_GBps"],
                                                 ceil["read2_write1_device_scope_GBps"])
    assert abs(ceil["frac_of_read2_write1"] - roof["achieved"] / ceil["read2_write1_best_GBps"]) < 1e-3
    assert abs(ceil["frac_of_read1_write1"] - roof["achieved"] / ceil["read1_write1_GBps"]) < 1e-3
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] == 1 and cpu["value"] > 0 and cpu["runs"] == 3
    assert len(d["inputs"]["sha256"]["W"]) == 64
    assert set(d["outputs_sha256"]) == {"q", "scales"}
    host = d["host"]
    assert host["cpu_model"] and host["nproc"] and host["torch"] and host["gpu"]


def test_two_kernel_workload_and_options():
    d = run_bench("--workload", "moe_bwd", "--no-extras", "--no-ceiling", "--no-cpu-baseline",
                  "--no-output-hash")
    assert d["config"]["workload"] == "moe_bwd_jagged"
    kernels = d["kernels"]
    assert len(kernels) == 2
    for k in kernels.values():
        check_kernel(k)
    slower = max(kernels.values(), key=lambda k: k["cold_us"]["median"])
    assert d["roofline"]["avg_launch_us"] == slower["cold_us"]["median"]
    assert d["workloads"] == {} and d["stream_ceiling"] is None and d["cpu_baseline"] is None
    assert d["vs_baseline"] is None and "baseline" not in d   # no page figure for this workload
    assert set(d["inputs"]["sha256"]) == {"grad_out_t", "x"}
