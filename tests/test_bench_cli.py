"""Host-side checks of bench.py's command line (no GPU needed)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert out["n_gpus"] == 2 and "one GPU" in out["error"]


def test_workload_table_names_every_configuration():
    sys.path.insert(0, ROOT)
    import bench

    for name in ("mx3d_e64", "moe_bwd", "moe_bwd_mx", "mx3d", "mx3d_rceil", "blockwise",
                 "blockwise_t", "relayout", "copy"):
        assert name in bench.WORKLOADS, name
    assert callable(bench.build)
    args = bench.parse([])
    assert args.workload == "mx3d_e64" and args.gpus == 1
    assert set(args.extras.split(",")) == {"moe_bwd", "moe_bwd_ws", "moe_bwd_g256_ws", "mx3d", "blockwise"}
