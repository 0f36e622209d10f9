"""The CPU oracle over the independent units of a full-size workload, in
parallel host processes.

Each unit is a complete reduction unit of the op: an expert of a 3D weight,
a block of rows of a rowwise operand (every (row, group) or 1 x B block lies
in one row), a block of columns of a colwise operand (every (group, column)
lies in one column), or a run of 128-row block rows for 128 x 128 blocks.
Put back together in order, the pieces are exactly the oracle's output for
the whole tensor: the oracle's loops never look past a unit.  The pool test
(``test_oracle_pool.py``) checks that on small inputs.

Test infrastructure: the workers load only ``oracle`` and ``workloads``.
Workers are spawned (not forked), so they never inherit a GPU context.
"""
from __future__ import annotations

import atexit
import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

# outputs of each oracle op, and the axis along which a unit split of the
# input splits them: rowwise-type ops split rows (axis 0) and their outputs
# along rows; colwise-type ops split columns (axis 1)
SPLIT_AXIS = {
    "quantize_jagged_rowwise": 0,
    "quantize_jagged_colwise": 1,
    "quantize_jagged_mx_rowwise": 0,
    "quantize_jagged_mx_colwise": 1,
    "quantize_mx_rowwise": 0,
    "quantize_blockwise": 0,
    "quantize_mx_3d_colwise": 0,
}

_pool = None


def workers() -> int:
    """Host processes to use: the cores this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def pool() -> ProcessPoolExecutor:
    global _pool
    if _pool is None:
        _pool = ProcessPoolExecutor(max_workers=workers(), mp_context=mp.get_context("spawn"))
        atexit.register(shutdown)
    return _pool


def shutdown() -> None:
    global _pool
    if _pool is not None:
        _pool.shutdown(wait=True, cancel_futures=True)
        _pool = None


def _run_op(name, x, kwargs):
    import oracle

    return getattr(oracle, name)(x, **kwargs)


def _bounds(n: int, parts: int, align: int):
    """Cut [0, n) into at most ``parts`` pieces on multiples of ``align``."""
    units = n // align
    parts = max(1, min(parts, units))
    cuts = [align * (units * k // parts) for k in range(parts + 1)]
    cuts[-1] = n
    return [(a, b) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]


def split_op(name: str, x: np.ndarray, *args, align: int = 1, parts: int = 0, axis=None,
             **kwargs):
    """``oracle.<name>(x, *args, **kwargs)`` computed on unit-aligned slices of
    x in parallel and put back together.  ``align``: the slice boundary
    granularity along the split axis (128 for 128-row blocks).  ``axis``:
    blockwise ops may also be split along columns (with ``align`` the
    block's column count); every output then splits along the same axis."""
    if axis is None:
        axis = SPLIT_AXIS[name]
    elif axis != SPLIT_AXIS[name] and name != "quantize_blockwise":
        raise ValueError(f"{name} splits along axis {SPLIT_AXIS[name]} only")
    n = x.shape[axis]
    parts = parts or 4 * workers()
    futs = []
    for a, b in _bounds(n, parts, align):
        sl = (slice(a, b), slice(None)) if axis == 0 else (slice(None), slice(a, b))
        piece = np.ascontiguousarray(x[sl])
        kw = dict(kwargs)
        for k, v in zip(_positional(name), args):
            kw[k] = v
        futs.append(pool().submit(_run_op, name, piece, kw))
    outs = [f.result() for f in futs]
    return tuple(np.concatenate([o[i] for o in outs], axis=axis) for i in range(len(outs[0])))


def _positional(name: str):
    return {"quantize_jagged_rowwise": ("offs",), "quantize_jagged_colwise": ("offs",),
            "quantize_jagged_mx_rowwise": ("offs",), "quantize_jagged_mx_colwise": ("offs",),
            "quantize_mx_rowwise": (), "quantize_blockwise": ("block_r", "block_c"),
            "quantize_mx_3d_colwise": ()}[name]


def _mx3d_expert_job(e: int, sweep: bool, modes, keep_bits: bool, shape):
    import oracle
    import workloads

    kw = {} if shape is None else {"N": shape[0], "K": shape[1]}
    bits = workloads.mx3d_sweep_expert(e, **kw) if sweep else workloads.mx3d_expert(e, **kw)
    out = {}
    for m in modes:
        q, s = oracle.quantize_mx_3d_colwise(bits[None], mode=m)
        out[m] = (q[0], s[0])
    return e, (bits if keep_bits else None), out


def mx3d_experts(experts, sweep: bool, modes=("floor",), keep_bits: bool = True, shape=None):
    """Yield (e, bf16 bits of expert e, {mode: (q (N, K), scales (N/32, K))})
    in expert order; each expert is generated and quantized by the oracle in
    a worker process.  ``shape``: (N, K) other than the workload's (8192,
    5120)."""
    # a bounded window of jobs in flight keeps at most that many experts'
    # results waiting in this process
    experts = [int(e) for e in experts]
    window = 2 * workers()
    futs = {}
    for i, e in enumerate(experts):
        futs[i] = pool().submit(_mx3d_expert_job, e, sweep, tuple(modes), keep_bits, shape)
        if i >= window:
            yield futs.pop(i - window).result()
    for i in sorted(futs):
        yield futs.pop(i).result()


def _encode_job(y):
    import oracle

    return oracle.e4m3_encode(y)


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """oracle.e4m3_encode over a 1-D array, in parallel chunks."""
    y = np.ascontiguousarray(y, dtype=np.float32).ravel()
    n = y.size
    futs = [pool().submit(_encode_job, y[a:b]) for a, b in _bounds(n, 4 * workers(), 1)]
    parts = [f.result() for f in futs]
    return np.concatenate(parts) if parts else np.empty(0, np.uint8)
