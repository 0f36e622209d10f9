"""A seeded random sweep of every entry point against the CPU oracle, byte
for byte: many small configurations drawn from a fixed seed (extents not
multiples of anything the kernels tile by, 1 to 100 groups with empty groups
and short tails, group starts on and off 8/16/32-element boundaries, both
scale modes, every layout with a kernel, the colwise call with and without
a workspace), adversarial bf16 values; bytes
past the last group keep the canary.  It adds breadth to the hand-picked
cases of the other parity tests."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (CANARY, DEV, adversarial, assert_same_bytes, bf16_dev, blockwise, colwise_workspace,
                         i32_dev, jagged_colwise, jagged_colwise_ws, jagged_mx_colwise, jagged_mx_rowwise,
                         jagged_rowwise, mx_3d_colwise, mx_rowwise, random_offsets, relayout)
import workloads

pytestmark = pytest.mark.gpu

N_CASES = 96


def _groups(g, extent):
    G = int(g.choice([1, 2, 3, 5, 8, 17, 64, 65, 100]))
    mult = int(g.choice([1, 8, 16, 32]))
    tail = int(g.integers(0, min(20, extent) + 1))
    seed = int(g.integers(1 << 30))
    if (extent - tail) // mult < 1:
        mult = 1
    return random_offsets(extent, G, seed, multiple=mult, short_tail=tail)


@pytest.mark.parametrize("k", range(N_CASES))
def test_jagged_fp32(k):
    g = np.random.default_rng([7101, k])
    rows, cols = int(g.integers(1, 300)), int(g.integers(1, 5000))
    bits = adversarial((rows, cols), 7200 + k)
    offs = _groups(g, cols)
    q, s = jagged_rowwise(bf16_dev(bits), i32_dev(offs))
    oq, os_ = oracle.quantize_jagged_rowwise(bits, offs, canary=CANARY)
    assert_same_bytes(q, oq, f"rowwise case {k} q")
    assert_same_bytes(s, os_, f"rowwise case {k} scales")

    rows, cols = int(g.integers(1, 6000)), 8 * int(g.integers(1, 65))
    bits = adversarial((rows, cols), 7300 + k)
    offs = _groups(g, rows)
    q, s = jagged_colwise(bf16_dev(bits), i32_dev(offs))
    oq, os_ = oracle.quantize_jagged_colwise(bits, offs, canary=CANARY)
    assert_same_bytes(q, oq, f"colwise case {k} q")
    assert_same_bytes(s, os_, f"colwise case {k} scales")
    # the same operand through the call with a workspace
    ws = colwise_workspace(rows, cols, len(offs))
    q, s = jagged_colwise_ws(bf16_dev(bits), i32_dev(offs), ws)
    assert_same_bytes(q, oq, f"colwise (workspace) case {k} q")
    assert_same_bytes(s, os_, f"colwise (workspace) case {k} scales")
    assert int(torch.count_nonzero(ws)) == 0, f"case {k}: workspace not left zero-filled"


@pytest.mark.parametrize("k", range(N_CASES))
def test_jagged_mx(k):
    g = np.random.default_rng([7102, k])
    mode = "rceil" if k % 2 else "floor"
    rows, cols = int(g.integers(1, 200)), int(g.integers(1, 5000))
    bits = adversarial((rows, cols), 7400 + k)
    offs = _groups(g, cols)
    q, s = jagged_mx_rowwise(bf16_dev(bits), i32_dev(offs), mode)
    oq, os_ = oracle.quantize_jagged_mx_rowwise(bits, offs, mode=mode, canary=CANARY)
    assert_same_bytes(q, oq, f"jagged mx rowwise case {k} q")
    assert_same_bytes(s, os_, f"jagged mx rowwise case {k} scales")

    rows, cols = int(g.integers(1, 5000)), 8 * int(g.integers(1, 40))
    bits = adversarial((rows, cols), 7500 + k)
    offs = _groups(g, rows)
    q, s = jagged_mx_colwise(bf16_dev(bits), i32_dev(offs), mode)
    oq, os_ = oracle.quantize_jagged_mx_colwise(bits, offs, mode=mode, canary=CANARY)
    assert_same_bytes(q, oq, f"jagged mx colwise case {k} q")
    assert_same_bytes(s, os_, f"jagged mx colwise case {k} scales")


@pytest.mark.parametrize("k", range(N_CASES))
def test_fixed_blocks(k):
    g = np.random.default_rng([7103, k])
    mode = "rceil" if k % 2 else "floor"
    E, N, K = int(g.integers(1, 4)), 32 * int(g.integers(1, 12)), 8 * int(g.integers(1, 80))
    w = adversarial((E, N, K), 7600 + k)
    q, s = mx_3d_colwise(bf16_dev(w), mode=mode)
    oq, os_ = oracle.quantize_mx_3d_colwise(w, mode=mode)
    assert_same_bytes(q, oq, f"mx3d case {k} q")
    assert_same_bytes(s, os_, f"mx3d case {k} scales")

    rows, cols = int(g.integers(1, 300)), 32 * int(g.integers(1, 100))
    x = adversarial((rows, cols), 7700 + k)
    q, s = mx_rowwise(bf16_dev(x), mode=mode)
    oq, os_ = oracle.quantize_mx_rowwise(x, mode=mode)
    assert_same_bytes(q, oq, f"mx rowwise case {k} q")
    assert_same_bytes(s, os_, f"mx rowwise case {k} scales")

    br, bc = [(1, 128), (128, 128), (128, 1)][k % 3]
    view = ("row_major", "transposed")[(k // 3) % 2]
    qlayout = ("row", "col")[(k // 6) % 2]
    # the tile kernel (every layout but 1 x 128 into row-major q) takes rows
    # in 16s; the transposed view swaps the roles of rows and columns
    m_r = 16 if br == 1 else br
    m_c = bc if bc == 128 else (16 if view == "transposed" and qlayout == "row" else 8)
    rows = m_r * int(g.integers(1, 40 if br == 1 else 5))
    cols = m_c * int(g.integers(1, 10 if bc == 128 else 60))
    x = adversarial((rows, cols), 7800 + k)
    dx = bf16_dev(x) if view == "row_major" else bf16_dev(np.ascontiguousarray(x.T)).t()
    q, s = blockwise(dx, br, bc, qlayout=qlayout)
    oq, os_ = oracle.quantize_blockwise(x, br, bc)
    assert_same_bytes(q, oq, f"blockwise {br}x{bc} {view} -> {qlayout} case {k} q")
    assert_same_bytes(s, os_, f"blockwise {br}x{bc} {view} -> {qlayout} case {k} scales")


@pytest.mark.parametrize("k", range(N_CASES))
def test_relayout(k):
    g = np.random.default_rng([7104, k])
    rows, extent = int(g.integers(1, 300)), int(g.integers(1, 60000))
    offs = _groups(g, extent)
    cap = oracle.jagged_mx_scale_capacity(extent, len(offs))
    layout = k % 3
    if layout == 0:      # blocks contiguous, row pitch off 16
        pitch = cap + int(g.integers(0, 9))
        host = workloads.e8m0_bytes((rows, pitch), 7900 + k)
        s_np, dev = host[:, :cap], torch.from_numpy(host).to(DEV)[:, :cap]
    elif layout == 1:    # rows contiguous (the colwise operand's transposed view)
        host = workloads.e8m0_bytes((cap, rows), 7900 + k)
        s_np, dev = host.T, torch.from_numpy(host).to(DEV).t()
    else:                # neither
        host = workloads.e8m0_bytes((rows, 3 * cap), 7900 + k)
        s_np, dev = host[:, ::3], torch.from_numpy(host).to(DEV)[:, ::3]
    t, st = relayout(dev, offs, extent)
    ot, ost = oracle.relayout_mx_scales_grouped(s_np, offs, extent, canary=CANARY)
    assert np.array_equal(st, ost), f"relayout case {k} tile starts"
    assert np.array_equal(t, ot), f"relayout case {k} tiles (layout {layout})"
