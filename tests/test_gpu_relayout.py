"""GPU parity of the per-group scale re-layout against the CPU oracle, byte
for byte: tiles, tile starts, and the bytes past the last tile (canary),
for the three input layouts (scales contiguous along blocks, along rows, or
neither), base pointers off every 4-byte alignment, ragged row counts, empty
groups, tokens past the last group, groups longer than one 8192-token item,
G on both sides of the one-wave table limit, and the full (8192, 32768)
scale shape.  Then the consumer side: a grouped GEMM on the real gfx950
scaled MFMA that reads the tiles reproduces the grouped GEMM of the
dequantized jagged MX operands, and agrees with the CPU model of the
instruction."""
import numpy as np
import pytest
import torch

import consumer
import mxfp8_quantization_moe_amd as mxq
import oracle
import workloads
from gpu_helpers import CANARY, DEV, i32_dev, random_offsets, relayout
from scaled_mfma_model import dequantized_gemm

pytestmark = pytest.mark.gpu


def check(scales_np, scales_dev, offs, extent, what):
    t, s = relayout(scales_dev, offs, extent)
    ot, os_ = oracle.relayout_mx_scales_grouped(scales_np, offs, extent, canary=CANARY)
    assert np.array_equal(s, os_), f"{what}: tile starts {s} vs {os_}"
    if not np.array_equal(t, ot):
        bad = np.flatnonzero(t != ot)
        raise AssertionError(f"{what}: {bad.size} tile bytes differ, first at {bad[0]} "
                             f"(tile {bad[0] // 256}, lane {(bad[0] % 256) // 4}, byte {bad[0] % 4}): "
                             f"{t[bad[0]]} vs {ot[bad[0]]}")


CASES = [
    # rows, extent, G, multiple, short tail, seed
    (37, 3000, 4, 1, 5, 1),
    (16, 512, 1, 1, 0, 2),
    (1, 20000, 7, 16, 0, 3),
    (200, 40000, 3, 32, 100, 4),        # groups spanning several 8192-token items
    (33, 70000, 300, 1, 9, 5),          # G > 64: workgroup-wide tables
    (5, 1000, 64, 1, 0, 6),             # G = 64: one-wave tables
    (5, 1000, 65, 1, 0, 7),
    (300, 6000, 8, 512, 0, 8),          # every group a whole number of tiles
]


@pytest.mark.parametrize("rows,extent,G,mult,tail,seed", CASES)
def test_block_contiguous_scales(rows, extent, G, mult, tail, seed):
    offs = random_offsets(extent, G, seed, multiple=mult, short_tail=tail)
    cap = oracle.jagged_mx_scale_capacity(extent, G)
    s = workloads.e8m0_bytes((rows, cap), 800 + seed)
    check(s, torch.from_numpy(s).to(DEV), offs, extent, "ss_b == 1")


@pytest.mark.parametrize("shift", [1, 2, 3])
def test_unaligned_base_and_pitch(shift):
    """Base pointer and row pitch off 4-byte alignment: each row's span
    starts at a different byte of its dword."""
    rows, extent, G = 45, 9000, 5
    offs = random_offsets(extent, G, 20 + shift, short_tail=3)
    cap = oracle.jagged_mx_scale_capacity(extent, G)
    big = workloads.e8m0_bytes((rows, cap + shift + 2), 830 + shift)
    view = torch.from_numpy(big).to(DEV)[:, shift:shift + cap]
    check(big[:, shift:shift + cap], view, offs, extent, f"shift {shift}")


@pytest.mark.parametrize("cols,extent,G,mult,tail,seed", [
    (24, 1300, 3, 1, 50, 11),
    (300, 9000, 6, 16, 0, 12),
    (16, 512, 1, 1, 0, 13),
    (4096, 16384, 8, 16, 0, 14),        # the MoE x operand's scales
    (77, 3000, 100, 1, 7, 15),
])
def test_row_contiguous_scales(cols, extent, G, mult, tail, seed):
    """The colwise operand: scales stored (blocks, cols) row-major, passed as
    the (cols, blocks) transposed view (ss_r == 1)."""
    offs = random_offsets(extent, G, seed, multiple=mult, short_tail=tail)
    cap = oracle.jagged_mx_scale_capacity(extent, G)
    s = workloads.e8m0_bytes((cap, cols), 840 + seed)
    view = torch.from_numpy(s).to(DEV).t()
    check(s.T, view, offs, extent, "ss_r == 1")


def test_other_strides():
    rows, extent, G = 21, 5000, 4
    offs = random_offsets(extent, G, 31, short_tail=2)
    cap = oracle.jagged_mx_scale_capacity(extent, G)
    big = workloads.e8m0_bytes((rows, 2 * cap), 850)
    view = torch.from_numpy(big).to(DEV)[:, ::2]
    check(big[:, ::2], view, offs, extent, "ss_b == 2")


def test_empty_extents():
    # no rows: only tile_starts (all zero) are written
    t, s = relayout(torch.zeros((0, 40), dtype=torch.uint8, device=DEV), [100, 300], 300)
    assert t.size == 0 and list(s) == [0, 0, 0]
    # no tokens: no tiles
    z = torch.zeros((20, 8), dtype=torch.uint8, device=DEV)
    t, s = relayout(z, [0, 0, 0], 0)
    assert list(s) == [0, 0, 0, 0]
    # offsets past the extent are clamped as in the jagged MX calls
    s_np = workloads.e8m0_bytes((20, 40), 860)
    t, st = relayout(torch.from_numpy(s_np).to(DEV), [300, 5000], 1000)
    ot, ost = oracle.relayout_mx_scales_grouped(s_np, [300, 1000], 1000, canary=CANARY)
    assert np.array_equal(st, ost) and np.array_equal(t, ot[:t.size])


def test_full_scale_shape():
    """(8192, 32768) scale columns, 8 MoE-like groups over 2^20 tokens."""
    s, offs = workloads.relayout_case()
    check(s, torch.from_numpy(s).to(DEV), offs, 1 << 20, "relayout (8192, 32768)")


# ------------------------------------------------------ the consumer side

def _spread(shape, seed, axis):
    g = workloads.rng(seed)
    v = g.standard_normal(shape).astype(np.float32)
    n, other = shape[axis], shape[1 - axis]
    e = g.integers(-8, 9, size=(other, (n + 7) // 8)).repeat(8, axis=1)[:, :n]
    v *= np.exp2(e if axis == 1 else e.T).astype(np.float32)
    return workloads.to_bf16_bits(v)


def _consume(qa, ta, sta, qb, tb, stb, offs, rows, cols):
    d = {k: torch.from_numpy(np.ascontiguousarray(v)).to(DEV)
         for k, v in dict(qa=qa, ta=ta, sta=sta, qb=qb, tb=tb, stb=stb,
                          offs=np.asarray(offs, np.int32)).items()}
    G = len(offs)
    nra, nrb = (rows + 15) // 16, (cols + 15) // 16
    out = torch.zeros((G, 16 * nra, 16 * nrb), dtype=torch.float32, device=DEV)
    rc = consumer.load().consumer_grouped_gemm(
        d["qa"].data_ptr(), qa.shape[1], rows, d["qb"].data_ptr(), qb.shape[1], cols,
        d["ta"].data_ptr(), d["sta"].data_ptr(), d["tb"].data_ptr(), d["stb"].data_ptr(),
        d["offs"].data_ptr(), G, out.data_ptr(), 0, nra, 0, nrb)
    assert rc == 0
    return out[:, :rows, :cols].cpu().numpy().astype(np.float64)


# The instruction does not accumulate like sequential IEEE fp32 additions:
# against exact float64 sums these cases are off by up to 6.7e-5 (~2^-14) of
# the sum of |terms| (measured), so the bound is 2^-11 of that sum.  A scale
# taken from the wrong block, row or K step changes a block's terms by a
# factor 2^k (k != 0 for almost every block of these inputs), an error above
# 2^-7 of the sum.
REL = 2.0 ** -11


def _abs_terms(qa, sa, qb, sb, offs):
    strip = lambda q: np.where(q >= 0x80, q - 0x80, q).astype(np.uint8)
    return dequantized_gemm(strip(qa), sa, strip(qb), sb, offs)


def _worst(got, want, absref):
    return max(float(np.max(np.abs(x - y) / (a + 1e-30))) for x, y, a in zip(got, want, absref))


def _tolerance_ok(got, want, qa, sa, qb, sb, offs):
    w = _worst(got, want, _abs_terms(qa, sa, qb, sb, offs))
    print(f"worst error / sum|terms| = {w:.3e} (bound {REL:.3e})")
    assert w <= REL, f"worst error {w:.3e} of the sum of |terms| (bound {REL:.3e})"


@pytest.mark.parametrize("rows,cols,extent,offs,seed", [
    (40, 24, 1300, [700, 700, 1250], 1),
    (16, 16, 1100, [33, 545, 1100], 2),
    (48, 32, 5000, [1000, 1000, 2100, 4999], 3),
])
def test_scaled_mfma_reads_the_oracle_tiles(rows, cols, extent, offs, seed):
    """The oracle's quantized operands and re-laid-out scales, consumed by
    the real instruction, give the dequantized grouped GEMM."""
    a = _spread((rows, extent), seed, 1)
    x = _spread((extent, cols), seed + 1, 0)
    qa, sa = oracle.quantize_jagged_mx_rowwise(a, offs)
    qx, sx = oracle.quantize_jagged_mx_colwise(x, offs)
    qb, sb = np.ascontiguousarray(qx.T), sx.T
    ta, sta = oracle.relayout_mx_scales_grouped(sa, offs, extent)
    tb, stb = oracle.relayout_mx_scales_grouped(sb, offs, extent)
    got = _consume(qa, ta, sta, qb, tb, stb, offs, rows, cols)
    want = dequantized_gemm(qa, sa, qb, sb, offs)
    _tolerance_ok(got, want, qa, sa, qb, sb, offs)
    # the same check sees a planted layout mistake: the four bytes of every
    # lane word reversed (K steps of a tile swapped) in A's tiles
    bad = ta.reshape(-1, 4)[:, ::-1].reshape(-1).copy()
    got_bad = _consume(qa, bad, sta, qb, tb, stb, offs, rows, cols)
    assert _worst(got_bad, want, _abs_terms(qa, sa, qb, sb, offs)) > 2.0 ** -7


def test_scaled_mfma_end_to_end_through_the_library():
    """Jagged MX quantization and re-layout on the device, consumed by the
    scaled MFMA: the same grouped GEMM as the oracle's operands give."""
    rows, cols, extent = 64, 48, 3000
    offs = [512, 512, 1700, 2990]
    a = _spread((rows, extent), 9, 1)
    x = _spread((extent, cols), 10, 0)
    d_offs = i32_dev(offs)
    to_dev = lambda b: torch.from_numpy(b.view(np.int16)).to(DEV).view(torch.bfloat16)
    qa, sa = mxq.quantize_jagged_mx_rowwise(to_dev(a), d_offs)
    qx, sx = mxq.quantize_jagged_mx_colwise(to_dev(x), d_offs)
    ta, sta = mxq.relayout_mx_scales_grouped(sa, d_offs, extent)
    tb, stb = mxq.relayout_mx_scales_grouped(sx.t(), d_offs, extent)
    qa_np = qa.view(torch.uint8).cpu().numpy()
    qb_np = np.ascontiguousarray(qx.view(torch.uint8).cpu().numpy().T)
    got = _consume(qa_np, ta.cpu().numpy(), sta.cpu().numpy(), qb_np, tb.cpu().numpy(),
                   stb.cpu().numpy(), offs, rows, cols)
    oqa, osa = oracle.quantize_jagged_mx_rowwise(a, offs)
    oqx, osx = oracle.quantize_jagged_mx_colwise(x, offs)
    oqb, osb = np.ascontiguousarray(oqx.T), osx.T
    want = dequantized_gemm(oqa, osa, oqb, osb, offs)
    _tolerance_ok(got, want, oqa, osa, oqb, osb, offs)


@pytest.mark.parametrize("layout", [0, 1, 2])
def test_maximum_group_count(layout):
    """G = 4096 (the ABI's limit), most groups empty or a few tokens long:
    the workgroup-wide tables, for each input layout."""
    G, extent, rows = 4096, 70000, 40
    offs = random_offsets(extent, G, 870 + layout, short_tail=3)
    cap = oracle.jagged_mx_scale_capacity(extent, G)
    if layout == 0:
        s = workloads.e8m0_bytes((rows, cap), 880)
        s_np, dev = s, torch.from_numpy(s).to(DEV)
    elif layout == 1:
        s = workloads.e8m0_bytes((cap, rows), 881)
        s_np, dev = s.T, torch.from_numpy(s).to(DEV).t()
    else:
        s = workloads.e8m0_bytes((rows, 2 * cap), 882)
        s_np, dev = s[:, ::2], torch.from_numpy(s).to(DEV)[:, ::2]
    check(s_np, dev, offs, extent, f"G = 4096, layout {layout}")


def test_scaled_mfma_at_the_moe_backward_shapes():
    """grad_out^T (4096, 16384) and x (16384, 4096) with the 8 MoE token
    groups, quantized and re-laid out on the device at full size; the real
    instruction consumes the tiles of the first and last two row blocks of
    each operand (tile numbers near both ends of every group's range) and
    reproduces the oracle's dequantized grouped GEMM of those rows and
    columns."""
    go = workloads.device_normal_bf16((4096, 16384), 31)
    x = workloads.device_normal_bf16((16384, 4096), 32)
    offs = workloads.moe_offsets()
    d_offs = i32_dev(offs)
    qa, sa = mxq.quantize_jagged_mx_rowwise(go, d_offs)
    qx, sx = mxq.quantize_jagged_mx_colwise(x, d_offs)
    ta, sta = mxq.relayout_mx_scales_grouped(sa, d_offs, 16384)
    tb, stb = mxq.relayout_mx_scales_grouped(sx.t(), d_offs, 16384)
    qa_u8 = qa.view(torch.uint8)
    qb_u8 = qx.view(torch.uint8).t()          # (cols, tokens) view of the column-major q
    G = offs.size
    lib = consumer.load()
    picks = [0, 1, 254, 255]                  # 16-row blocks sampled from each operand
    rows_a = np.concatenate([np.arange(16 * b, 16 * b + 16) for b in picks])
    rows_b = rows_a
    idx = torch.from_numpy(rows_a).to(DEV)
    a_bits = go.index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)
    x_bits = np.ascontiguousarray(
        x.index_select(1, torch.from_numpy(rows_b).to(DEV)).view(torch.int16).cpu().numpy().view(np.uint16))
    oqa, osa = oracle.quantize_jagged_mx_rowwise(a_bits, offs)
    oqx, osx = oracle.quantize_jagged_mx_colwise(x_bits, offs)
    oqb, osb = np.ascontiguousarray(oqx.T), osx.T
    want = dequantized_gemm(oqa, osa, oqb, osb, offs)           # G x (64, 64)
    absref = _abs_terms(oqa, osa, oqb, osb, offs)
    for ia, ba in enumerate(picks):
        for ib, bb in enumerate(picks):
            out = torch.zeros((G, 16, 16), dtype=torch.float32, device=DEV)
            rc = lib.consumer_grouped_gemm(qa_u8.data_ptr(), qa_u8.stride(0), 4096,
                                           qb_u8.data_ptr(), qb_u8.stride(0), 4096,
                                           ta.data_ptr(), sta.data_ptr(), tb.data_ptr(),
                                           stb.data_ptr(), d_offs.data_ptr(), G, out.data_ptr(),
                                           ba, 1, bb, 1)
            assert rc == 0
            got = out.cpu().numpy().astype(np.float64)
            sl = (slice(16 * ia, 16 * ia + 16), slice(16 * ib, 16 * ib + 16))
            w = _worst(list(got), [m[sl] for m in want], [m[sl] for m in absref])
            assert w <= REL, f"row blocks {ba}, {bb}: worst {w:.3e} of the sum of |terms|"
