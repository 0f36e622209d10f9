"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no quantization arithmetic: it only draws random numbers
(numpy PCG64 streams from fixed ``SeedSequence`` seeds), rounds them once to
bf16 (round-to-nearest-even, through torch's float32 -> bfloat16 cast) and
returns the bf16 *bit patterns* as ``numpy.uint16`` arrays, plus int32 group
offsets.  Both the CPU oracle and the HIP library consume exactly these bytes.

Workloads (shapes and value distributions follow the MoE shapes the pages
benchmark: the (E, 8192, 5120) expert-weight sweep of the 3D colwise kernel
page, and the token-grouped operands of the jagged scaling pages):

* ``small``   A (256, 1024) rowwise and B (1024, 256) colwise, 4 groups of
              16-multiples summing to 1024, exactly one empty; N(0, 1).
* ``moe_bwd`` grad_out^T (4096, 16384) rowwise and x (16384, 4096) colwise,
              8 token groups (16-multiples, one empty, one >= 4096 long);
              N(0,1) x per-row lognormal(0, 2) x (100 with prob 1e-4).
* ``mx3d``    W (E, 8192, 5120), N(0, 0.02), one stream per expert.
* ``mx3d_sweep`` the same with 1% of 32x1 blocks zeroed and 1% scaled 2^20.
* ``blockwise`` act (8192, 4096) and W (4096, 4096), N(0,1) with 1/8 of the
              columns Student-t(3).
* ``relayout`` e8m0 scale bytes (8192, 32768 + 7) (uniform codes 0..254) for
              8 MoE-like token groups over 2^20 tokens: the largest scale
              shape of the per-group scale conversion benchmarks.
* ``large``   tensors of more than 2^31 elements (64-bit indexing checks),
              N(0,1) drawn directly on the GPU by torch's seeded Philox
              generator (too large to draw on the host in a test); the
              tests copy the bit patterns of sampled rows or columns back
              for the oracle.
"""
from __future__ import annotations

import numpy as np

try:  # torch is plumbing here: it provides the bf16 rounding cast
    import torch
except ImportError:  # pragma: no cover
    torch = None


# --------------------------------------------------------------- primitives

def rng(seed) -> np.random.Generator:
    if isinstance(seed, np.random.SeedSequence):
        return np.random.default_rng(seed)
    return np.random.default_rng(np.random.SeedSequence(seed))


def to_bf16_bits(f32: np.ndarray) -> np.ndarray:
    """Round float32 values once to bf16 (RNE) and return the uint16 bits."""
    f32 = np.ascontiguousarray(f32, dtype=np.float32)
    t = torch.from_numpy(f32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (for generators/tests)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def normal_bf16(shape, seed, std: float = 1.0) -> np.ndarray:
    g = rng(seed)
    v = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return to_bf16_bits(v)


# ---------------------------------------------------------------- offsets

def offsets_small(seed, extent: int = 1024, groups: int = 4) -> np.ndarray:
    """4 groups, sizes multiples of 16 summing to ``extent``, exactly one empty."""
    g = rng(seed)
    units = extent // 16
    j0 = int(g.integers(groups))
    nonempty = groups - 1
    extra = g.multinomial(units - nonempty, [1.0 / nonempty] * nonempty)
    sizes = np.zeros(groups, dtype=np.int64)
    k = 0
    for j in range(groups):
        if j == j0:
            continue
        sizes[j] = 16 * (1 + int(extra[k]))
        k += 1
    return np.cumsum(sizes).astype(np.int32)


def offsets_moe(seed, tokens: int = 16384, groups: int = 8) -> np.ndarray:
    """8 token groups in units of 16 tokens: one empty group, one group that
    receives 256 extra units (>= 4096 tokens), the rest split by a
    Dirichlet-weighted multinomial."""
    g = rng(seed)
    units = tokens // 16
    j0 = int(g.integers(groups))
    j1 = int(g.integers(groups - 1))
    if j1 >= j0:
        j1 += 1
    others = [j for j in range(groups) if j != j0]
    bulk = units - 256
    w = g.dirichlet(np.ones(len(others)))
    share = g.multinomial(bulk, w)
    u = np.zeros(groups, dtype=np.int64)
    for j, s in zip(others, share):
        u[j] = int(s)
    u[j1] += 256
    assert u.sum() == units
    return np.cumsum(16 * u).astype(np.int32)


# --------------------------------------------------------------- workloads

SMALL_SEEDS = dict(a_offs=1101, a_vals=1102, b_offs=1103, b_vals=1104)
MOE_SEEDS = dict(offs=2101, go_vals=2102, x_vals=2103)
MX3D_SEED = 3101
MX3D_SWEEP_SEEDS = dict(vals=4101, pattern=4102)
BLOCKWISE_SEEDS = dict(act_vals=5101, act_tcols=5102, w_vals=5103, w_tcols=5104)


def small_rowwise():
    """(A bits (256, 1024), offs int32[4]) — groups along dim 1."""
    return normal_bf16((256, 1024), SMALL_SEEDS["a_vals"]), offsets_small(SMALL_SEEDS["a_offs"])


def small_colwise():
    """(B bits (1024, 256), offs int32[4]) — groups along dim 0."""
    return normal_bf16((1024, 256), SMALL_SEEDS["b_vals"]), offsets_small(SMALL_SEEDS["b_offs"])


def _moe_values(shape, seed) -> np.ndarray:
    g = rng(seed)
    rows, cols = shape
    z = g.standard_normal(size=shape, dtype=np.float32)
    row_mult = np.exp(2.0 * g.standard_normal(size=(rows, 1))).astype(np.float32)
    z *= row_mult
    outlier = g.random(size=shape, dtype=np.float32) < np.float32(1e-4)
    z[outlier] *= np.float32(100.0)
    return to_bf16_bits(z)


def moe_offsets() -> np.ndarray:
    return offsets_moe(MOE_SEEDS["offs"])


# per-group shifts of the MoE group ends (the last end stays at the extent):
# starts off 8- and 16-element boundaries
MOE_END_SHIFTS = (0, 3, 5, 5, 1, 7, 2, 0)


def moe_offsets_unaligned(extent: int = 16384) -> np.ndarray:
    """The MoE group ends moved by MOE_END_SHIFTS (ends 6016, 8947, 9189,
    9189, 10113, 13671, 14322, 16384 at 16384 tokens)."""
    return np.minimum(moe_offsets() + np.array(MOE_END_SHIFTS), extent).astype(np.int32)


MOE_FINE_SEED = 2104


def offsets_fine(seed, tokens: int = 16384, groups: int = 256) -> np.ndarray:
    """Many token groups (a fine-grained MoE layer) in units of 16 tokens:
    multinomial shares with Dirichlet(4) weights, so sizes spread around
    tokens / groups and a few groups are empty."""
    g = rng(seed)
    units = tokens // 16
    share = g.multinomial(units, g.dirichlet(np.full(groups, 4.0)))
    return (np.cumsum(share) * 16).astype(np.int32)


def moe_offsets_fine(groups: int = 256) -> np.ndarray:
    return offsets_fine(MOE_FINE_SEED, groups=groups)


def moe_grad_out_t() -> np.ndarray:
    """grad_out^T (4096, 16384) bits, row-major; groups along dim 1."""
    return _moe_values((4096, 16384), MOE_SEEDS["go_vals"])


def moe_x() -> np.ndarray:
    """x (16384, 4096) bits, row-major; groups along dim 0."""
    return _moe_values((16384, 4096), MOE_SEEDS["x_vals"])


def mx3d_expert(e: int, N: int = 8192, K: int = 5120, num_streams: int = 8) -> np.ndarray:
    """Expert e of W (E, N, K), N(0, 0.02)."""
    ss = np.random.SeedSequence(MX3D_SEED).spawn(num_streams)[e]
    return normal_bf16((N, K), ss, std=0.02)


def mx3d_sweep_expert(e: int, N: int = 8192, K: int = 5120) -> np.ndarray:
    """Expert e of the E sweep: N(0, 0.02) with 1% of the 32x1 blocks all +0.0
    and 1% multiplied by 2^20 (exact).  Experts are prefixes: W_E = W_64[:E]."""
    vs = np.random.SeedSequence(MX3D_SWEEP_SEEDS["vals"]).spawn(64)[e]
    ps = np.random.SeedSequence(MX3D_SWEEP_SEEDS["pattern"]).spawn(64)[e]
    v = rng(vs).standard_normal(size=(N, K), dtype=np.float32)
    v *= np.float32(0.02)
    u = rng(ps).random(size=(N // 32, K), dtype=np.float32)
    zero = np.repeat(u < np.float32(0.01), 32, axis=0)
    big = np.repeat((u >= np.float32(0.01)) & (u < np.float32(0.02)), 32, axis=0)
    v[zero] = np.float32(0.0)
    v[big] *= np.float32(2.0 ** 20)
    return to_bf16_bits(v)


def _heavy_tailed(shape, vals_seed, tcols_seed) -> np.ndarray:
    rows, cols = shape
    v = rng(vals_seed).standard_normal(size=shape, dtype=np.float32)
    gt = rng(tcols_seed)
    tcols = np.sort(gt.choice(cols, size=cols // 8, replace=False))
    v[:, tcols] = gt.standard_t(3, size=(rows, tcols.size)).astype(np.float32)
    return to_bf16_bits(v)


def blockwise_act() -> np.ndarray:
    """act (8192, 4096) bits; quantized in 1x128 blocks."""
    s = BLOCKWISE_SEEDS
    return _heavy_tailed((8192, 4096), s["act_vals"], s["act_tcols"])


def blockwise_weight() -> np.ndarray:
    """W (4096, 4096) bits; quantized in 128x128 blocks."""
    s = BLOCKWISE_SEEDS
    return _heavy_tailed((4096, 4096), s["w_vals"], s["w_tcols"])


# ----------------------------------------------------------- byte accounting

RELAYOUT_SEEDS = dict(offs=6101, scales=6102)


def e8m0_bytes(shape, seed) -> np.ndarray:
    """Random e8m0 scale bytes (codes 0..254; 255 is the NaN code)."""
    return rng(seed).integers(0, 255, size=shape, dtype=np.uint8)


def relayout_case(rows: int = 8192, tokens: int = 1 << 20, groups: int = 8):
    """Scales of ``rows`` rows for jagged MX blocks over ``tokens`` tokens in
    ``groups`` MoE-like token groups (offsets_moe: multiples of 16, one empty
    group, one long group): returns (scales (rows, capacity) uint8, offs).
    The default is the largest scale shape of the per-group conversion
    benchmarks, (8192, 32768) scale columns."""
    offs = offsets_moe(RELAYOUT_SEEDS["offs"], tokens=tokens, groups=groups)
    cap = (tokens + 31) // 32 + groups - 1
    return e8m0_bytes((rows, cap), RELAYOUT_SEEDS["scales"]), offs


def algorithmic_bytes(numel: int, scale_bytes: int) -> int:
    """bf16 read + e4m3 write + scale write (offsets excluded)."""
    return 2 * numel + numel + scale_bytes


def device_normal_bf16(shape, seed: int, device="cuda"):
    """N(0,1) bf16 tensor drawn on the GPU with torch's seeded generator.
    For inputs too large to draw on the host; callers hand the oracle the
    bit patterns of whatever part they check, read back from the device."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
