"""Pins of the oracle's re-layout of jagged MX scales into scaled-MFMA scale
tiles ("[mxfp8 moe training] add CUDA kernel for per-group conversion of scale
factors to blocked layout": per-group conversion for groups along K; the
page leaves the target layout to the consumer).

The layout has no printed definition to compare against, so it is pinned
from the consumer's side: a grouped GEMM computed by a CPU model of the
gfx950 scaled MFMA (``scaled_mfma_model``, written from the instruction's
operand order) reading the re-laid-out scales must equal the grouped GEMM
of the dequantized jagged MX operands, for groups of every alignment,
empty groups, a ragged row count and tokens past the last group.  A
transposed tile, a swapped byte or lane index, a wrong tile order or a
wrong group base changes that product.  The GPU consumer test runs the same
check with the real instruction.  Structural pins: the valid entries of each
group are a permutation of its scales, padding is zero, bytes past the last
tile are untouched, and the tile counts follow from the group sizes.
"""
import numpy as np
import pytest

import oracle
import workloads
from scaled_mfma_model import dequantized_gemm, grouped_gemm


def _spread(shape, seed, axis):
    """N(0,1) times 2^e, e in [-8, 8] drawn per 8 tokens along ``axis`` and
    per row, so neighbouring 32-token blocks get different e8m0 codes and a
    scale applied to the wrong block shows in the product."""
    g = workloads.rng(seed)
    v = g.standard_normal(shape).astype(np.float32)
    n = shape[axis]
    other = shape[1 - axis]
    e = g.integers(-8, 9, size=(other, (n + 7) // 8)).repeat(8, axis=1)[:, :n]
    v *= np.exp2(e if axis == 1 else e.T).astype(np.float32)
    return workloads.to_bf16_bits(v)


def _operands(rows, cols, extent, offs, seed):
    a = _spread((rows, extent), seed, 1)
    x = _spread((extent, cols), seed + 1, 0)
    qa, sa = oracle.quantize_jagged_mx_rowwise(a, offs)
    qx, sx = oracle.quantize_jagged_mx_colwise(x, offs)
    return qa, sa, np.ascontiguousarray(qx.T), sx.T


@pytest.mark.parametrize("rows,cols,extent,offs,seed", [
    (40, 24, 1300, [700, 700, 1250], 1),      # ragged rows, empty group, tokens past the end
    (16, 16, 1100, [33, 545, 1100], 2),       # starts off every 32 / 128 / 512 boundary
    (20, 18, 2100, [2100], 3),                # one group, several scale tiles
])
def test_consumer_model_reproduces_the_dequantized_grouped_gemm(rows, cols, extent, offs, seed):
    qa, sa, qb, sb = _operands(rows, cols, extent, offs, seed)
    ta, sta = oracle.relayout_mx_scales_grouped(sa, offs, extent)
    tb, stb = oracle.relayout_mx_scales_grouped(sb, offs, extent)
    got = grouped_gemm(qa, ta, sta, qb, tb, stb, offs)
    want = dequantized_gemm(qa, sa, qb, sb, offs)
    for g, (x, y) in enumerate(zip(got, want)):
        assert x.shape == y.shape == (rows, cols)
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-30, err_msg=f"group {g}")


def test_consumer_model_sees_a_swapped_tile_order():
    """The pin is sensitive: the same tiles read column-major (kt-major)
    instead of row-block-major give a different product."""
    rows, cols, extent, offs = 32, 16, 1100, [1100]
    qa, sa, qb, sb = _operands(rows, cols, extent, offs, 4)
    ta, sta = oracle.relayout_mx_scales_grouped(sa, offs, extent)
    tb, stb = oracle.relayout_mx_scales_grouped(sb, offs, extent)
    kt, rb = 3, 2
    swapped = ta.copy()
    for r in range(rb):
        for k in range(kt):
            src = (r * kt + k) * 256
            dst = (k * rb + r) * 256
            swapped[dst:dst + 256] = ta[src:src + 256]
    good = grouped_gemm(qa, ta, sta, qb, tb, stb, offs)[0]
    bad = grouped_gemm(qa, swapped, sta, qb, tb, stb, offs)[0]
    want = dequantized_gemm(qa, sa, qb, sb, offs)[0]
    np.testing.assert_allclose(good, want, rtol=1e-12)
    assert not np.allclose(bad, want, rtol=1e-6)


def _structure(scales, offs, extent, canary=0xA5):
    rows = scales.shape[0]
    out, starts = oracle.relayout_mx_scales_grouped(scales, offs, extent, canary=canary)
    RB = (rows + 15) // 16
    sizes = np.diff(np.concatenate([[0], np.asarray(offs)]))
    nbs = [(int(n) + 31) // 32 for n in sizes]
    kts = [(nb + 15) // 16 for nb in nbs]
    assert list(starts) == list(np.concatenate([[0], np.cumsum([RB * k for k in kts])]))
    assert out.size == oracle.mx_tile_capacity(rows, extent, len(offs))
    assert np.all(out[starts[-1] * 256:] == canary)
    b0 = 0
    for g, (nb, kt) in enumerate(zip(nbs, kts)):
        region = out[starts[g] * 256:starts[g + 1] * 256]
        valid = scales[:, b0:b0 + nb]
        # one 16 x 16 window of the scale matrix per tile, so the multiset of
        # each tile is its window's multiset plus zero padding
        for r in range(RB):
            for k in range(kt):
                tile = region[(r * kt + k) * 256:(r * kt + k + 1) * 256]
                win = valid[16 * r:16 * r + 16, 16 * k:16 * k + 16]
                pad = 256 - win.size
                assert np.array_equal(np.sort(tile),
                                      np.sort(np.concatenate([win.reshape(-1),
                                                              np.zeros(pad, np.uint8)])))
        b0 += nb
    return out, starts


def test_structure_and_padding():
    g = np.random.default_rng(7)
    rows, extent = 37, 3000
    offs = [100, 100, 1700, 2990]
    cap = oracle.jagged_mx_scale_capacity(extent, len(offs))
    scales = g.integers(1, 255, size=(rows, cap)).astype(np.uint8)
    _structure(scales, offs, extent)
    # a strided (transposed) view gives the same bytes as its contiguous copy
    t = np.ascontiguousarray(scales.T).T
    a, _ = _structure(t, offs, extent)
    b, _ = oracle.relayout_mx_scales_grouped(np.ascontiguousarray(scales), offs, extent, canary=0xA5)
    assert np.array_equal(a, b)


def test_first_tile_of_a_full_group():
    """16 rows, one 512-token group: lane word 16j + i holds row i's blocks
    j, 4 + j, 8 + j, 12 + j (one per K step of 128 tokens)."""
    s = (np.arange(16)[:, None] * 16 + np.arange(16)[None, :]).astype(np.uint8)
    out, starts = oracle.relayout_mx_scales_grouped(s, [512], 512)
    words = out[:256].reshape(64, 4)
    for lane in range(64):
        j, i = divmod(lane, 16)
        assert list(words[lane]) == [s[i, 4 * u + j] for u in range(4)]
    assert list(starts) == [0, 1]


def test_no_rows_and_empty_groups():
    out, starts = oracle.relayout_mx_scales_grouped(np.zeros((0, 10), np.uint8), [40, 300], 300)
    assert out.size == 0 and list(starts) == [0, 0, 0]
    out, starts = oracle.relayout_mx_scales_grouped(np.full((5, 4), 9, np.uint8), [0, 0, 0], 64,
                                                    canary=3)
    assert list(starts) == [0, 0, 0, 0] and np.all(out == 3)
