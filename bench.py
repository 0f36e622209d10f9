#!/usr/bin/env python3
"""Throughput benchmark of the fp8 quantization hot path on one MI355X.

Default workload (``mx3d_e64``): MXFP8 quantization of 3D expert weights W
bf16 (64, 8192, 5120) along N in 32 x 1 blocks (e8m0 floor scales), written
per expert column-major, the largest configuration and the shape of the 3D
colwise kernel page's headline row; values N(0, 0.02) with 1% of the blocks
all-zero and 1% scaled by 2^20.  One step = one launch over all 64 experts.

Other workloads (``--workload``): ``moe_bwd`` (jagged rowwise quantization
of grad_out^T (4096, 16384) plus jagged colwise of x (16384, 4096), 8 token
groups, fp32 scales), ``moe_bwd_ws`` (the colwise operand with a workspace), ``moe_bwd_g256`` and
``moe_bwd_g256_ws`` (the same operands in the 256 token groups of a
fine-grained MoE layer), ``moe_bwd_mx`` (the same operands as jagged MXFP8),
``mx3d`` (E = 8, N(0, 0.02)), ``mx3d_e{1,2,4,16,64}`` (the E sweep),
``mx3d_rceil``, ``rowwise_g64`` (the jagged rowwise operand with 64 groups of
256 columns), ``moe_bwd_mx_unaligned`` (both jagged MX operands with group starts off
8- and 16-element boundaries), ``blockwise`` (1 x 128 activations (8192, 4096) + 128 x 128
weights (4096, 4096)), ``blockwise_t`` (the transposed operands of the
blockwise backward), ``relayout`` (per-group re-layout of (8192, 32768)
e8m0 scales into scaled-MFMA tiles), ``copy`` (counter calibration).

Metric: algorithmic HBM bytes (2 B bf16 read + 1 B e4m3 write + scale
bytes per launch) divided by time.  Inputs are resident in HBM before the
timed region; outputs are preallocated; every launch goes through the C ABI.

Timing:
  * ``value`` / ``ms_per_step``: K steps back to back, host clock, bracketed
    by synchronisations; ``gpu_ms_per_step``: one pair of HIP events on the
    launch stream around the same K steps.
  * per kernel, ``cold_us``: a 1 GiB write on the launch stream (more than
    the L2s and the 256 MB memory-side cache), then one event pair around one
    launch; median, min and max over ``--flush-iters`` launches.  The
    roofline uses the dominant kernel's cold median.
  * per kernel, ``warm_us``: one event pair around K back-to-back launches
    of that kernel alone, divided by K (inputs partly in the caches when they
    fit).
The extra workloads (``--extras``, default the MoE jagged operands without
and with a workspace, the same operands in 256 fine-grained token groups
with a workspace, the E=8 MX 3D weights and the blockwise operands) are
timed the same way and reported under ``workloads``; the
streaming probes under ``stream_ceiling`` give the practical HBM ceiling of
the same traffic mix.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0
# The pages' own figures for the MX 3D colwise quantization of (E, 8192, 5120)
# bf16 weights (the 3D CUDA kernel, Kernel microbenchmarks table of "[mxfp8
# moe training] add CUDA kernel to quantize 3d tensor colwise"), in the same
# byte model (2 B read + 1 B written per element + 1/32 B of e8m0 scales),
# measured on another vendor's GPU: the reference point of vs_baseline, not a
# target.
PAGE_MX3D_GBPS = {1: 525.128, 2: 1018.23, 4: 1710.16, 8: 2462.8, 16: 3304.82, 64: 4152.11}
PAGE_MX3D_SOURCE = ("3D CUDA kernel on (E, 8192, 5120), Kernel microbenchmarks table of \"[mxfp8 moe training] "
                    "add CUDA kernel to quantize 3d tensor colwise\"; other hardware")


def page_baseline(workload: str):
    """The pages' GB/s for this workload's shape and metric, or None."""
    if workload == "mx3d":
        return PAGE_MX3D_GBPS[8]
    if workload.startswith("mx3d_e") and workload[len("mx3d_e"):].isdigit():
        return PAGE_MX3D_GBPS.get(int(workload[len("mx3d_e"):]))
    return None
METRIC = "achieved HBM GB/s (bf16 read + fp8/scale write) and % of MI355X peak"
DEFAULT_EXTRAS = "moe_bwd,moe_bwd_ws,moe_bwd_g256_ws,mx3d,blockwise"
FLUSH_BYTES = 1 << 30


def parse(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="mx3d_e64")
    p.add_argument("--flush-iters", type=int, default=10,
                   help="cold launches per kernel, each after a 1 GiB write (median/min/max)")
    p.add_argument("--extras", default=DEFAULT_EXTRAS,
                   help="comma-separated extra workloads timed after the headline one")
    p.add_argument("--no-extras", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-ceiling", action="store_true",
                   help="skip the device copy and the streaming probes")
    p.add_argument("--no-output-hash", action="store_true")
    p.add_argument("--gen-workers", type=int, default=-1,
                   help="host processes drawing the inputs (-1: one per core, at most 16; 0: draw "
                        "in this process, e.g. under a profiler that would follow child processes)")
    return p.parse_args(argv)


def csrc_digest() -> str:
    """Digest of the kernel sources with comments and blank space removed, so
    the counter summary stays valid across comment-only edits."""
    import re

    d = os.path.join(ROOT, "mxfp8_quantization_moe_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        with open(os.path.join(d, name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = "\n".join(line.strip() for line in text.splitlines() if line.strip())
        h.update(name.encode())
        h.update(text.encode())
    return h.hexdigest()[:16]


# ----------------------------------------------------- input generation

def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _gen_call(name, args):
    import workloads

    return getattr(workloads, name)(*args)


class Generator:
    """Seeded inputs from ``workloads``, drawn in spawned host processes
    (numpy only: no GPU context), with the SHA-256 of every tensor's bytes
    in the order they are handed over."""

    def __init__(self, workers: int = -1):
        self._pool = None
        self.workers = _workers() if workers < 0 else workers
        self.sha = {}

    def pool(self):
        if self._pool is None:
            import multiprocessing as mp
            from concurrent.futures import ProcessPoolExecutor

            self._pool = ProcessPoolExecutor(max_workers=self.workers, mp_context=mp.get_context("spawn"))
        return self._pool

    def map(self, name, arglist, label):
        """Yield workloads.<name>(*args) for each args in order, hashing the
        concatenated bytes under ``label``."""
        h = hashlib.sha256()
        if self.workers == 0:
            results = (_gen_call(name, tuple(a)) for a in arglist)
        else:
            futs = [self.pool().submit(_gen_call, name, tuple(a)) for a in arglist]
            results = (f.result() for f in futs)
        for out in results:
            h.update(memoryview(out).cast("B"))
            yield out
        self.sha[label] = h.hexdigest()

    def one(self, name, label, *args):
        return next(iter(self.map(name, [args], label)))

    def close(self):
        if self._pool is not None:
            self._pool.shutdown(wait=True)
            self._pool = None


# ------------------------------------------------------------- workloads

class Launch:
    """One C-ABI call with preallocated device buffers."""

    def __init__(self, name, kernel, fn, args, nbytes, numel, outputs=()):
        self.name, self.kernel, self.fn, self.args = name, kernel, fn, args
        self.nbytes, self.numel = nbytes, numel
        self.outputs = outputs   # (label, device tensor) whose bytes are hashed

    def __call__(self, stream_handle):
        code = self.fn(*self.args, stream_handle)
        if code != 0:
            raise RuntimeError(f"{self.name}: status {code}")


def bf16_dev(torch, bits):
    import numpy as np

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _sizes(offs):
    import numpy as np

    return [int(v) for v in np.diff(np.concatenate([[0], offs]))]


def build_moe_bwd(torch, mxq, workloads, gen, ws=False, fine=False):
    """ws: the colwise operand through the call with a workspace (long token
    groups split across workgroups, every element read once).  fine: 256
    token groups of a fine-grained MoE layer (sizes multiples of 16 around
    64, some empty) instead of the 8 MoE groups."""
    go_t, x = list(gen.map("moe_grad_out_t", [()], "grad_out_t")) + list(gen.map("moe_x", [()], "x"))
    offs = workloads.moe_offsets_fine() if fine else workloads.moe_offsets()
    G = offs.size
    d_go, d_x = bf16_dev(torch, go_t), bf16_dev(torch, x)
    d_offs = torch.from_numpy(offs).cuda()
    R1, C1 = go_t.shape
    R2, C2 = x.shape
    q1 = torch.empty(R1 * C1, dtype=torch.uint8, device="cuda")
    s1 = torch.empty(R1 * G, dtype=torch.float32, device="cuda")
    q2 = torch.empty(R2 * C2, dtype=torch.uint8, device="cuda")
    s2 = torch.empty(G * C2, dtype=torch.float32, device="cuda")
    keep = [d_go, d_x, d_offs, q1, s1, q2, s2]
    l1 = Launch("jagged_rowwise grad_out^T (4096,16384)",
                "jagged_contig_seg_kernel<8>" if G > 1 else "jagged_contig_kernel<8>",
                mxq.mxq_quantize_jagged_rowwise,
                (d_go.data_ptr(), R1, C1, C1, 1, d_offs.data_ptr(), G, q1.data_ptr(), C1, 1,
                 s1.data_ptr(), G, 1), 3 * R1 * C1 + 4 * R1 * G, R1 * C1, (("q1", q1), ("s1", s1)))
    cargs = (d_x.data_ptr(), R2, C2, C2, 1, d_offs.data_ptr(), G, q2.data_ptr(), 1, R2, s2.data_ptr(), C2, 1)
    # the colwise tile kernel takes one-tile chunks for groups of at most 128
    # rows on average, two-tile chunks otherwise
    tile_kernel = "jagged_colwise_tile_kernel<%d>" % (1 if R2 <= 128 * G else 2)
    if ws:
        nws = mxq.mxq_jagged_colwise_workspace_bytes(R2, C2, G)
        d_ws = torch.zeros(max(nws, 4) // 4, dtype=torch.int32, device="cuda")
        keep.append(d_ws)
        l2 = Launch("jagged_colwise (workspace) x (16384,4096)", tile_kernel,
                    mxq.mxq_quantize_jagged_colwise_ws, cargs + (d_ws.data_ptr(), nws),
                    3 * R2 * C2 + 4 * G * C2, R2 * C2, (("q2", q2), ("s2", s2)))
    else:
        # two launches: jagged_colwise_tile_clear_kernel zeroes the long
        # groups' scale slots, then the tile kernel exchanges maxima through them
        l2 = Launch("jagged_colwise x (16384,4096), clear + tile", tile_kernel,
                    mxq.mxq_quantize_jagged_colwise, cargs,
                    3 * R2 * C2 + 4 * G * C2, R2 * C2, (("q2", q2), ("s2", s2)))
    desc = {"workload": "moe_bwd_jagged" + ("_g256" if fine else "") + ("_ws" if ws else ""),
            "tensors": "grad_out^T bf16 (4096,16384) rowwise -> row-major e4m3; "
                       "x bf16 (16384,4096) colwise -> column-major e4m3",
            "groups": int(G), "group_sizes": _sizes(offs),
            "scales": "fp32 per (row, group) and per (group, column)",
            "seeds": dict(workloads.MOE_SEEDS, **({"offs": workloads.MOE_FINE_SEED} if fine else {}))}

    def cpu_sample(oracle):
        n = 1024
        nbytes = 3 * n * C1 + 4 * n * G + 3 * R2 * n + 4 * G * n
        xs = x[:, :n].copy()
        return (lambda: (oracle.quantize_jagged_rowwise(go_t[:n], offs),
                         oracle.quantize_jagged_colwise(xs, offs)),
                nbytes, f"jagged rowwise on {n} of 4096 rows of grad_out^T and jagged colwise on "
                        f"{n} of 4096 columns of x (all 16384 tokens, same {G} groups)")

    return [l1, l2], keep, desc, cpu_sample


def build_rowwise_groups(torch, mxq, workloads, gen, G=64):
    """Jagged rowwise quantization of grad_out^T (4096, 16384) with G equal
    token groups (64 groups of 256 columns by default): the many-groups
    kernel."""
    import numpy as np

    go_t = gen.one("moe_grad_out_t", "grad_out_t")
    R, C = go_t.shape
    offs = (np.arange(1, G + 1) * (C // G)).astype(np.int32)
    d_go = bf16_dev(torch, go_t)
    d_offs = torch.from_numpy(offs).cuda()
    q = torch.empty(R * C, dtype=torch.uint8, device="cuda")
    s = torch.empty(R * G, dtype=torch.float32, device="cuda")
    l = Launch(f"jagged_rowwise grad_out^T (4096,16384), {G} groups", "jagged_contig_seg_kernel<8>",
               mxq.mxq_quantize_jagged_rowwise,
               (d_go.data_ptr(), R, C, C, 1, d_offs.data_ptr(), G, q.data_ptr(), C, 1, s.data_ptr(), G, 1),
               3 * R * C + 4 * R * G, R * C, (("q", q), ("s", s)))
    desc = {"workload": f"rowwise_g{G}", "tensors": "grad_out^T bf16 (4096,16384) rowwise -> row-major e4m3",
            "groups": G, "group_sizes": [C // G] * G, "scales": "fp32 per (row, group)",
            "seeds": {"go_vals": workloads.MOE_SEEDS["go_vals"]}}
    return [l], [d_go, d_offs, q, s], desc, None


def build_moe_bwd_mx(torch, mxq, workloads, gen, unaligned=False):
    """The MX variant of the MoE backward grad_weight operands: jagged MXFP8
    (32-element blocks restarting at each token-group start, e8m0 floor
    scales) of grad_out^T rowwise and x colwise, the same 8 groups.  With
    ``unaligned`` the group ends move by a few tokens (ends 6016, 8947,
    9189, 9189, 10113, 13671, 14322, 16384): group starts off 8- and
    16-element boundaries, so blocks start anywhere in a 16-byte chunk."""
    go_t, x = list(gen.map("moe_grad_out_t", [()], "grad_out_t")) + list(gen.map("moe_x", [()], "x"))
    offs = workloads.moe_offsets_unaligned() if unaligned else workloads.moe_offsets()
    G = offs.size
    d_go, d_x = bf16_dev(torch, go_t), bf16_dev(torch, x)
    d_offs = torch.from_numpy(offs).cuda()
    R1, C1 = go_t.shape
    R2, C2 = x.shape
    nb1 = mxq.jagged_mx_scale_capacity(C1, G)
    nb2 = mxq.jagged_mx_scale_capacity(R2, G)
    nb = int(sum((n + 31) // 32 for n in _sizes(offs)))          # blocks actually written
    q1 = torch.empty(R1 * C1, dtype=torch.uint8, device="cuda")
    s1 = torch.empty(R1 * nb1, dtype=torch.uint8, device="cuda")
    q2 = torch.empty(R2 * C2, dtype=torch.uint8, device="cuda")
    s2 = torch.empty(nb2 * C2, dtype=torch.uint8, device="cuda")
    keep = [d_go, d_x, d_offs, q1, s1, q2, s2]
    off = ", starts off 8" if unaligned else ""
    l1 = Launch(f"jagged_mx_rowwise grad_out^T (4096,16384){off}", "jagged_mx_rowwise_kernel<8>",
                mxq.mxq_quantize_jagged_mx_rowwise,
                (d_go.data_ptr(), R1, C1, C1, 1, d_offs.data_ptr(), G, q1.data_ptr(), C1, 1,
                 s1.data_ptr(), nb1, 1, 0), 3 * R1 * C1 + R1 * nb, R1 * C1, (("q1", q1),))
    l2 = Launch(f"jagged_mx_colwise x (16384,4096){off}", "jagged_mx_colwise_kernel",
                mxq.mxq_quantize_jagged_mx_colwise,
                (d_x.data_ptr(), R2, C2, C2, 1, d_offs.data_ptr(), G, q2.data_ptr(), 1, R2,
                 s2.data_ptr(), C2, 1, 0), 3 * R2 * C2 + nb * C2, R2 * C2, (("q2", q2),))
    desc = {"workload": "moe_bwd_jagged_mx_unaligned" if unaligned else "moe_bwd_jagged_mx",
            "tensors": "grad_out^T bf16 (4096,16384) 1x32 blocks per group -> row-major e4m3; "
                       "x bf16 (16384,4096) 32x1 blocks per group -> column-major e4m3",
            "groups": int(G), "group_sizes": _sizes(offs),
            "scales": f"e8m0 floor, {nb} blocks per row / column", "seeds": dict(workloads.MOE_SEEDS)}

    def cpu_sample(oracle):
        import numpy as np

        n = 1024
        xs = np.ascontiguousarray(x[:, :n])
        return (lambda: (oracle.quantize_jagged_mx_rowwise(go_t[:n], offs),
                         oracle.quantize_jagged_mx_colwise(xs, offs)),
                3 * n * C1 + n * nb + 3 * R2 * n + nb * n,
                f"jagged MX rowwise on {n} of 4096 rows of grad_out^T and jagged MX colwise on "
                f"{n} of 4096 columns of x")

    return [l1, l2], keep, desc, cpu_sample


def build_mx3d(torch, mxq, workloads, gen, E, sweep, rceil=False):
    import numpy as np

    N, K = 8192, 5120
    w = torch.empty((E, N, K), dtype=torch.bfloat16, device="cuda")
    name = "mx3d_sweep_expert" if sweep else "mx3d_expert"
    first = []   # the oracle's sample: the first (up to) three experts
    for e, bits in enumerate(gen.map(name, [(e,) for e in range(E)], "W")):
        w[e].copy_(bf16_dev(torch, bits))
        if e < 3:
            first.append(bits)
        if E > 8 and (e + 1) % 16 == 0:
            print(f"[bench] {e + 1} of {E} experts on the device", file=sys.stderr, flush=True)
    q = torch.empty(E * N * K, dtype=torch.uint8, device="cuda")
    s = torch.empty(E * (N // 32) * K, dtype=torch.uint8, device="cuda")
    l = Launch(f"mx_3d_colwise ({E},{N},{K})", "block_strided_kernel<32, 1, true, false>",
               mxq.mxq_quantize_mx_3d_colwise,
               (w.data_ptr(), E, N, K, N * K, K, 1, q.data_ptr(), N * K, 1, N, s.data_ptr(),
                (N // 32) * K, K, 1, 1 if rceil else 0), 3 * E * N * K + E * (N // 32) * K, E * N * K,
               (("q", q), ("scales", s)))
    mode = "rceil" if rceil else "floor"
    seeds = dict(workloads.MX3D_SWEEP_SEEDS) if sweep else {"vals": workloads.MX3D_SEED}
    desc = {"workload": f"mx3d_E{E}" + ("_sweep" if sweep else "") + ("_rceil" if rceil else ""),
            "tensors": f"W bf16 ({E},{N},{K}) -> e4m3 per-expert column-major (N*K,1,N)",
            "values": "N(0,0.02)" + (", 1% of 32x1 blocks zero, 1% x 2^20" if sweep else ""),
            "scales": f"e8m0 {mode}, (E, N/32, K)", "seeds": seeds}

    sample = np.stack(first)
    ns = sample.shape[0]

    def cpu_sample(oracle):
        return (lambda: oracle.quantize_mx_3d_colwise(sample, mode=mode),
                ns * (3 * N * K + (N // 32) * K), f"experts 0-{ns - 1} of W, whole ({ns},{N},{K})")

    return [l], [w, q, s], desc, cpu_sample


def build_blockwise(torch, mxq, workloads, gen):
    a = gen.one("blockwise_act", "act")
    wt = gen.one("blockwise_weight", "W")
    da, dw = bf16_dev(torch, a), bf16_dev(torch, wt)
    M, Kd = a.shape
    R, C = wt.shape
    qa = torch.empty(M * Kd, dtype=torch.uint8, device="cuda")
    sa = torch.empty(M * (Kd // 128), dtype=torch.float32, device="cuda")
    qw = torch.empty(R * C, dtype=torch.uint8, device="cuda")
    sw = torch.empty((R // 128) * (C // 128), dtype=torch.float32, device="cuda")
    l1 = Launch("blockwise 1x128 act (8192,4096)", "block_contig_kernel<128, 8, false, 4>",
                mxq.mxq_quantize_blockwise,
                (da.data_ptr(), M, Kd, Kd, 1, 1, 128, qa.data_ptr(), Kd, 1, sa.data_ptr(),
                 Kd // 128, 1), 3 * M * Kd + 4 * M * (Kd // 128), M * Kd, (("qa", qa), ("sa", sa)))
    l2 = Launch("blockwise 128x128 W (4096,4096)", "block_strided_kernel<128, 128, false, false>",
                mxq.mxq_quantize_blockwise,
                (dw.data_ptr(), R, C, C, 1, 128, 128, qw.data_ptr(), 1, R, sw.data_ptr(),
                 C // 128, 1), 3 * R * C + 4 * (R // 128) * (C // 128), R * C, (("qw", qw), ("sw", sw)))
    desc = {"workload": "blockwise",
            "tensors": "act bf16 (8192,4096) 1x128 -> row-major e4m3; "
                       "W bf16 (4096,4096) 128x128 -> column-major e4m3",
            "scales": "fp32 per block", "seeds": dict(workloads.BLOCKWISE_SEEDS)}

    def cpu_sample(oracle):
        n = 2048
        return (lambda: (oracle.quantize_blockwise(a[:n], 1, 128), oracle.quantize_blockwise(wt[:n], 128, 128)),
                3 * n * Kd + 4 * n * (Kd // 128) + 3 * n * C + 4 * (n // 128) * (C // 128),
                f"{n} rows of act and {n} rows of W")

    return [l1, l2], [da, dw, qa, sa, qw, sw], desc, cpu_sample


def build_blockwise_t(torch, mxq, workloads, gen):
    """The transposed operands of the blockwise backward, read in place: the
    activations' 128 x 1 blocks of the (4096, 8192) transposed view into a
    row-major q of the transpose (scales per 128 tokens of each column), and
    the weights' 128 x 128 blocks of the transposed view into a row-major q."""
    a = gen.one("blockwise_act", "act")
    wt = gen.one("blockwise_weight", "W")
    da, dw = bf16_dev(torch, a), bf16_dev(torch, wt)
    M, Kd = a.shape
    R, C = wt.shape
    qa = torch.empty(M * Kd, dtype=torch.uint8, device="cuda")
    sa = torch.empty((M // 128) * Kd, dtype=torch.float32, device="cuda")
    qw = torch.empty(R * C, dtype=torch.uint8, device="cuda")
    sw = torch.empty((R // 128) * (C // 128), dtype=torch.float32, device="cuda")
    # act^T: a (Kd, M) view with strides (1, Kd); 1 x 128 blocks along its rows
    # are 128 x 1 blocks of act; q of act^T row-major (Kd, M)
    l1 = Launch("blockwise 1x128 act^T (4096,8192) view", "block_strided_kernel<128, 1, false, false>",
                mxq.mxq_quantize_blockwise,
                (da.data_ptr(), Kd, M, 1, Kd, 1, 128, qa.data_ptr(), M, 1, sa.data_ptr(),
                 M // 128, 1), 3 * M * Kd + 4 * Kd * (M // 128), M * Kd, (("qa", qa), ("sa", sa)))
    l2 = Launch("blockwise 128x128 W^T (4096,4096) view", "block_strided_kernel<128, 128, false, false>",
                mxq.mxq_quantize_blockwise,
                (dw.data_ptr(), C, R, 1, C, 128, 128, qw.data_ptr(), R, 1, sw.data_ptr(),
                 R // 128, 1), 3 * R * C + 4 * (R // 128) * (C // 128), R * C, (("qw", qw), ("sw", sw)))
    desc = {"workload": "blockwise_t",
            "tensors": "act^T view of bf16 (8192,4096) 1x128 -> row-major e4m3 (4096,8192); "
                       "W^T view of bf16 (4096,4096) 128x128 -> row-major e4m3",
            "scales": "fp32 per block", "seeds": dict(workloads.BLOCKWISE_SEEDS)}
    return [l1, l2], [da, dw, qa, sa, qw, sw], desc, None


def build_relayout(torch, mxq, workloads, gen):
    """Per-group re-layout of jagged MX scales into scaled-MFMA scale tiles on
    the largest scale shape of the per-group conversion benchmarks:
    (8192, 32768) e8m0 scale columns of 8 MoE-like token groups over 2^20
    tokens, stored row-major (blocks contiguous)."""
    scales, offs = workloads.relayout_case()
    gen.sha["scales"] = hashlib.sha256(memoryview(scales).cast("B")).hexdigest()
    rows, cap = scales.shape
    extent = 1 << 20
    G = offs.size
    sizes = _sizes(offs)
    nb = int(sum((n + 31) // 32 for n in sizes))
    ntiles = ((rows + 15) // 16) * int(sum((n + 511) // 512 for n in sizes))
    d_s = torch.from_numpy(scales).cuda()
    d_offs = torch.from_numpy(offs).cuda()
    tiles = torch.empty(mxq.mx_tile_capacity(rows, extent, G), dtype=torch.uint8, device="cuda")
    starts = torch.empty(G + 1, dtype=torch.int32, device="cuda")
    l = Launch(f"relayout_mx_scales ({rows},{nb}) e8m0, {G} groups", "relayout_mx_scales_kernel<0, 4, false>",
               mxq.mxq_relayout_mx_scales_grouped,
               (d_s.data_ptr(), rows, cap, 1, d_offs.data_ptr(), G, extent, tiles.data_ptr(),
                starts.data_ptr()), rows * nb + 256 * ntiles, rows * nb)
    desc = {"workload": "relayout_scales",
            "tensors": f"e8m0 scales ({rows},{nb}) row-major -> 16x16-block scaled-MFMA tiles "
                       f"({ntiles} tiles of 256 B)",
            "groups": int(G), "group_sizes": sizes,
            "bytes": "scale bytes read + tile bytes written (zero padding included)",
            "seeds": dict(workloads.RELAYOUT_SEEDS)}

    def cpu_sample(oracle):
        n = 2048
        nt = ((n + 15) // 16) * int(sum((v + 511) // 512 for v in sizes))
        return (lambda: oracle.relayout_mx_scales_grouped(scales[:n], offs, extent),
                n * nb + 256 * nt, f"{n} of {rows} rows, all {G} groups")

    return [l], [d_s, d_offs, tiles, starts], desc, cpu_sample


def build_copy(torch, mxq, workloads, gen):
    """Calibration: a plain device-to-device copy of 256 MiB (torch's copy,
    i.e. the runtime's copy kernel).  Its FETCH_SIZE / WRITE_SIZE counters
    against the known 256 MiB read and written give the scale factors that
    turn those counters into HBM bytes."""
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)

    class CopyLaunch(Launch):
        def __call__(self, stream_handle):
            dst.copy_(src)

    l = CopyLaunch("d2d copy 256 MiB", "copyBuffer", None, (), 2 * n, n)
    desc = {"workload": "copy_256MiB", "tensors": "uint8 256 MiB -> 256 MiB (calibration)"}
    return [l], [src, dst], desc, None


WORKLOADS = ("mx3d_e64", "mx3d_e1", "mx3d_e2", "mx3d_e4", "mx3d_e16", "mx3d", "mx3d_rceil",
             "moe_bwd", "moe_bwd_ws", "moe_bwd_g256", "moe_bwd_g256_ws", "moe_bwd_mx",
             "moe_bwd_mx_unaligned", "rowwise_g64", "blockwise",
             "blockwise_t", "relayout", "copy")


def build(name, torch, mxq, workloads, gen):
    if name == "copy":
        return build_copy(torch, mxq, workloads, gen)
    if name == "moe_bwd":
        return build_moe_bwd(torch, mxq, workloads, gen)
    if name == "moe_bwd_ws":
        return build_moe_bwd(torch, mxq, workloads, gen, ws=True)
    if name == "moe_bwd_g256":
        return build_moe_bwd(torch, mxq, workloads, gen, fine=True)
    if name == "moe_bwd_g256_ws":
        return build_moe_bwd(torch, mxq, workloads, gen, ws=True, fine=True)
    if name == "moe_bwd_mx":
        return build_moe_bwd_mx(torch, mxq, workloads, gen)
    if name == "moe_bwd_mx_unaligned":
        return build_moe_bwd_mx(torch, mxq, workloads, gen, unaligned=True)
    if name.startswith("rowwise_g") and name[len("rowwise_g"):].isdigit():
        return build_rowwise_groups(torch, mxq, workloads, gen, int(name[len("rowwise_g"):]))
    if name == "mx3d":
        return build_mx3d(torch, mxq, workloads, gen, 8, sweep=False)
    if name == "mx3d_rceil":
        return build_mx3d(torch, mxq, workloads, gen, 8, sweep=False, rceil=True)
    if name.startswith("mx3d_e") and name[len("mx3d_e"):].isdigit():
        return build_mx3d(torch, mxq, workloads, gen, int(name[len("mx3d_e"):]), sweep=True)
    if name == "blockwise":
        return build_blockwise(torch, mxq, workloads, gen)
    if name == "blockwise_t":
        return build_blockwise_t(torch, mxq, workloads, gen)
    if name == "relayout":
        return build_relayout(torch, mxq, workloads, gen)
    raise SystemExit(f"unknown workload {name}")


# -------------------------------------------------------------------- run

def traffic_for(kernel_name: str, workload: str):
    """HBM bytes per launch of `kernel_name` in `workload` from the committed
    rocprofv3 counter summary (profiles/traffic.json), if it was taken on the
    current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    if data.get("csrc_digest") != csrc_digest():
        return None
    for key, entry in data.get("kernels", {}).items():
        wl, _, kern = key.partition(":")
        if wl == workload and kern.startswith("mxq::" + kernel_name):
            return entry.get("hbm_bytes_per_launch")
    return None


class DeviceEvents:
    """Timing events on the launch stream with a device-scope release
    (hipEventReleaseToDevice), else without the system-scope fence
    (hipEventDisableSystemFence): recording them writes back and invalidates
    no caches for the host, so they perturb the kernels between them less
    than default events.  Uses the HIP runtime torch has already loaded (the
    one the launches go through)."""

    KINDS = ((0x40000000, "hipEventReleaseToDevice"), (0x20000000, "hipEventDisableSystemFence"))

    def __init__(self):
        lib = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD)
        lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        for f in (lib.hipEventCreateWithFlags, lib.hipEventRecord, lib.hipEventElapsedTime,
                  lib.hipEventDestroy):
            f.restype = ctypes.c_int
        self.lib = lib
        self.made = []
        self.flags, self.kind = None, None
        for flags, kind in self.KINDS:
            e = ctypes.c_void_p()
            if lib.hipEventCreateWithFlags(ctypes.byref(e), flags) == 0:
                lib.hipEventDestroy(e)
                self.flags, self.kind = flags, kind
                break
        if self.flags is None:
            raise OSError("no timing event kind accepted")

    def create(self):
        e = ctypes.c_void_p()
        if self.lib.hipEventCreateWithFlags(ctypes.byref(e), self.flags) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.made.append(e)
        return e

    def record(self, e, stream_handle):
        if self.lib.hipEventRecord(e, ctypes.c_void_p(stream_handle)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for e in self.made:
            self.lib.hipEventDestroy(e)
        self.made = []


class Timer:
    """Cold (flushed) and warm timings of single launches on one stream."""

    def __init__(self, torch, dev, sh):
        self.torch, self.dev, self.sh = torch, dev, sh
        self.flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")

    def cold_ms(self, fn, iters):
        pairs = [(self.dev.create(), self.dev.create()) for _ in range(iters)]
        for k, (a, b) in enumerate(pairs):
            self.flush.fill_(k & 0xFF)          # on the launch stream (torch's current stream)
            self.dev.record(a, self.sh)
            fn(self.sh)
            self.dev.record(b, self.sh)
        self.torch.cuda.synchronize()
        return [self.dev.elapsed_ms(a, b) for a, b in pairs]

    def warm_ms(self, fn, k):
        a, b = self.dev.create(), self.dev.create()
        fn(self.sh)
        self.dev.record(a, self.sh)
        for _ in range(k):
            fn(self.sh)
        self.dev.record(b, self.sh)
        self.torch.cuda.synchronize()
        return self.dev.elapsed_ms(a, b) / k


def kernel_record(np, l, cold, warm_ms):
    med = float(np.median(cold))
    return {"cold_us": {"median": round(med * 1e3, 2), "min": round(float(np.min(cold)) * 1e3, 2),
                        "max": round(float(np.max(cold)) * 1e3, 2), "iters": len(cold)},
            "warm_us": round(warm_ms * 1e3, 2),
            "algorithmic_bytes": l.nbytes,
            "GBps_cold": round(l.nbytes / (med * 1e-3) / 1e9, 1),
            "frac_of_peak_cold": round(l.nbytes / (med * 1e-3) / 1e9 / PEAK_GBPS, 4),
            "GBps_warm": round(l.nbytes / (warm_ms * 1e-3) / 1e9, 1),
            "kernel": l.kernel}


def time_kernels(np, timer, launches, flush_iters, warm_steps, warmup):
    for _ in range(max(1, warmup)):
        for l in launches:
            l(timer.sh)
    timer.torch.cuda.synchronize()
    out = {}
    for l in launches:
        cold = timer.cold_ms(l, flush_iters)
        out[l.name] = kernel_record(np, l, cold, timer.warm_ms(l, warm_steps))
    return out


def output_sha256(torch, launches):
    """SHA-256 of each launch's output buffers (storage order), copied back in
    64 MiB pieces."""
    res = {}
    for l in launches:
        for label, t in l.outputs:
            h = hashlib.sha256()
            flat = t.view(torch.uint8).reshape(-1)
            step = 64 << 20
            for i in range(0, flat.numel(), step):
                h.update(memoryview(flat[i:i + step].cpu().numpy()).cast("B"))
            res[label] = h.hexdigest()
    return res


def stream_ceiling(torch, dev, sh, np):
    """Practical HBM ceiling of the quantizers' traffic: the streaming probes
    (tests/ceiling: 2 reads : 1 write with nontemporal stores and with
    nontemporal device-scope stores, read only, write only, 1 read : 1 write)
    on 2^31 bf16 elements (4 GiB read, 2 or 4 GiB written), median of 5
    launches each, and the runtime's 4 GiB device-to-device copy."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import ceiling

    lib = ceiling.load()
    n = 1 << 31
    src = torch.empty(2 * n, dtype=torch.uint8, device="cuda").fill_(0x3C)
    dst = torch.empty(2 * n, dtype=torch.uint8, device="cuda")   # the 1:1 probe writes 2n bytes
    res = {"elements": n, "method": "event pair per launch, median of 5 (buffers far larger than the caches)"}
    for mode, code in ceiling.MODES.items():
        def fn(s, code=code):
            rc = lib.ceiling_stream(src.data_ptr(), dst.data_ptr(), n, code, ctypes.c_void_p(s))
            if rc != 0:
                raise RuntimeError(f"ceiling_stream mode {code}: {rc}")
        fn(sh)
        torch.cuda.synchronize()
        ms = []
        for _ in range(5):
            a, b = dev.create(), dev.create()
            dev.record(a, sh)
            fn(sh)
            dev.record(b, sh)
            torch.cuda.synchronize()
            ms.append(dev.elapsed_ms(a, b))
        res[f"{mode}_GBps"] = round(ceiling.bytes_moved(n, mode) / (float(np.median(ms)) * 1e-3) / 1e9, 1)
    del src, dst
    # the runtime's own copy kernel, counted as bytes read plus bytes written
    m = 4 << 30
    a8 = torch.empty(m, dtype=torch.uint8, device="cuda").fill_(1)
    b8 = torch.empty(m, dtype=torch.uint8, device="cuda")
    b8.copy_(a8)
    torch.cuda.synchronize()
    ms = []
    for _ in range(5):
        a, b = dev.create(), dev.create()
        dev.record(a, sh)
        b8.copy_(a8)
        dev.record(b, sh)
        torch.cuda.synchronize()
        ms.append(dev.elapsed_ms(a, b))
    res["d2d_copy_GBps"] = round(2 * m / (float(np.median(ms)) * 1e-3) / 1e9, 1)
    del a8, b8
    return res


def cpu_baseline(np, oracle, cpu_sample):
    """The oracle on a bounded sample of the workload, pinned to one host core
    (the calling thread's affinity), median of 3 runs."""
    fn, nbytes, what = cpu_sample(oracle)
    prev = None
    core = None
    try:
        prev = os.sched_getaffinity(0)
        core = min(prev)
        os.sched_setaffinity(0, {core})
    except (AttributeError, OSError):
        prev = None
    try:
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn()
            times.append(time.perf_counter() - t0)
    finally:
        if prev is not None:
            os.sched_setaffinity(0, prev)
    dt = float(np.median(times))
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": what, "seconds_median": round(dt, 3), "runs": 3,
            "pinned_core": core, "bytes": nbytes}


def host_info(torch):
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = None
    rocm = None
    for p in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        if os.path.exists(p):
            rocm = open(p).read().strip()
            break
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity_cores": affinity,
            "gpu": torch.cuda.get_device_name(0), "torch": torch.__version__,
            "hip": getattr(torch.version, "hip", None), "rocm": rocm, "python": platform.python_version()}


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        raise SystemExit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) != 1:
        raise SystemExit("one process, one GPU: run without torch.distributed")

    import numpy as np
    import torch

    import mxfp8_quantization_moe_amd as mxq
    import workloads

    mxq._capi.load()
    torch.cuda.init()
    dev = DeviceEvents()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    gen = Generator(args.gen_workers)
    print(f"[bench] building workload {args.workload}", file=sys.stderr, flush=True)
    launches, keep, desc, cpu_sample = build(args.workload, torch, mxq, workloads, gen)
    input_sha = dict(gen.sha)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        for l in launches:
            l(sh)
    torch.cuda.synchronize()

    # timed region: K steps exactly as a caller runs them, bracketed by one
    # pair of events on the launch stream (none between launches)
    K = args.steps
    g0, g1 = dev.create(), dev.create()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    dev.record(g0, sh)
    for _ in range(K):
        for l in launches:
            l(sh)
    dev.record(g1, sh)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = dev.elapsed_ms(g0, g1)
    print(f"[bench] timed {K} steps: {wall * 1e3 / K:.4f} ms per step", file=sys.stderr, flush=True)

    timer = Timer(torch, dev, sh)
    kernels = time_kernels(np, timer, launches, args.flush_iters, K, 0)
    out_sha = None if args.no_output_hash else output_sha256(torch, launches)

    step_bytes = sum(l.nbytes for l in launches)
    ms_per_step = wall * 1e3 / K
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    dom = max(launches, key=lambda l: kernels[l.name]["cold_us"]["median"])
    dk = kernels[dom.name]
    achieved = dom.nbytes / (dk["cold_us"]["median"] * 1e-6) / 1e9
    traffic = traffic_for(dom.kernel, args.workload)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic, "kernel": dom.kernel,
            "algorithmic_bytes_per_launch": dom.nbytes,
            "avg_launch_us": dk["cold_us"]["median"],
            "timing": f"cold: 1 GiB write, then {dev.kind} events around one launch; "
                      f"median of {args.flush_iters}"}
    del keep, launches

    extras = {}
    if not args.no_extras:
        for name in [n for n in args.extras.split(",") if n and n != args.workload]:
            print(f"[bench] extra workload {name}", file=sys.stderr, flush=True)
            gen.sha = {}
            ls, kp, d, _ = build(name, torch, mxq, workloads, gen)
            torch.cuda.synchronize()
            extras[d["workload"]] = {"config": d, "input_sha256": dict(gen.sha),
                                     "kernels": time_kernels(np, timer, ls, args.flush_iters, K, 2)}
            del ls, kp
            torch.cuda.empty_cache()
    gen.close()
    del timer
    torch.cuda.empty_cache()

    ceiling = None
    if not args.no_ceiling:
        print("[bench] streaming ceiling", file=sys.stderr, flush=True)
        ceiling = stream_ceiling(torch, dev, sh, np)
        # the faster of the two 2:1 probes (nontemporal stores, or nontemporal
        # at device scope) is the ceiling the kernel is held to
        best = max(ceiling["read2_write1_GBps"], ceiling["read2_write1_device_scope_GBps"])
        ceiling["read2_write1_best_GBps"] = best
        ceiling["frac_of_read2_write1"] = round(achieved / best, 4)
        ceiling["frac_of_read1_write1"] = round(achieved / ceiling["read1_write1_GBps"], 4)
        ceiling["frac_of_d2d_copy"] = round(achieved / ceiling["d2d_copy_GBps"], 4)

    cpu = None
    if not args.no_cpu_baseline and cpu_sample is not None:
        import oracle

        print("[bench] timing the CPU oracle on a sample (one core, 3 runs)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(np, oracle, cpu_sample)

    desc = dict(desc)
    desc["io"] = "bf16 in; e4m3 q and e8m0 or fp32 scales out; fp32 arithmetic"
    base = page_baseline(args.workload)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "gpu_ms_per_step": round(gpu_ms / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / base, 4) if base else None,
        "dtype": "f32",
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / PEAK_GBPS, 2),
        "config": desc,
        "roofline": roof,
        "kernels": kernels,
        "workloads": extras,
        "stream_ceiling": ceiling,
        "cpu_baseline": cpu,
        "inputs": {"sha256": input_sha, "generator": "numpy PCG64 SeedSequence, rounded once to bf16 (RNE)"},
        "outputs_sha256": out_sha,
        "host": host_info(torch),
        "csrc_digest": csrc_digest(),
    }
    if base:
        out["baseline"] = {"value": base, "unit": "GB/s", "source": PAGE_MX3D_SOURCE}
    print(json.dumps(out), flush=True)
    dev.close()


if __name__ == "__main__":
    main()
