"""GPU parity of every C-ABI entry point against the CPU oracle, byte for
byte, on small and adversarial inputs: ragged group boundaries, empty groups,
offsets that stop short of the extent (bytes past the last group must keep
the canary), single groups, many groups, tails that are not tile multiples,
zero / subnormal / huge MX blocks, transposed views, a side stream, and
repeat-run determinism."""
import numpy as np
import pytest
import torch

import mxfp8_quantization_moe_amd as mxq
import oracle
import oracle_pool
import workloads
from gpu_helpers import (CANARY, adversarial, assert_same_bytes, bf16_dev, blockwise, i32_dev,
                         jagged_colwise, jagged_rowwise, mx_3d_colwise, mx_rowwise, random_offsets)

pytestmark = pytest.mark.gpu


def check_rowwise(bits, offs, canary_tail=True):
    q, s = jagged_rowwise(bf16_dev(bits), i32_dev(offs))
    oq, os_ = oracle.quantize_jagged_rowwise(bits, offs, canary=CANARY)
    assert_same_bytes(q, oq, "jagged rowwise q")
    assert_same_bytes(s, os_, "jagged rowwise scales")


def check_colwise(bits, offs):
    q, s = jagged_colwise(bf16_dev(bits), i32_dev(offs))
    oq, os_ = oracle.quantize_jagged_colwise(bits, offs, canary=CANARY)
    assert_same_bytes(q, oq, "jagged colwise q")
    assert_same_bytes(s, os_, "jagged colwise scales")


# ------------------------------------------------------------------ jagged

def test_small_workloads():
    a, offs = workloads.small_rowwise()
    check_rowwise(a, offs)
    b, offs_b = workloads.small_colwise()
    check_colwise(b, offs_b)


@pytest.mark.parametrize("rows,cols,G,mult,tail,seed", [
    (5, 1000, 4, 1, 0, 1),
    (3, 4099, 7, 1, 5, 2),
    (2, 20000, 8, 16, 0, 3),       # longer than the register window: chunked re-read
    (9, 40000, 13, 1, 33, 4),
    (4, 77, 1, 1, 0, 5),
    (6, 300, 64, 1, 0, 6),
    (2, 5000, 300, 1, 7, 7),       # many groups: binary-search group lookup
    (3, 9000, 4096, 1, 0, 30),     # the most groups, most of them empty
    (1, 1, 2, 1, 0, 8),
    (7, 8, 3, 1, 1, 9),
    (8, 16384, 17, 1, 0, 40),      # many groups off 8-column boundaries, full register window
    (8, 16384, 64, 1, 0, 41),
    (8, 16384, 64, 16, 3, 42),
    (2000, 16384, 33, 8, 0, 43),   # more rows than workgroups: each walks several rows
    (1500, 12000, 100, 1, 5, 44),
    (4, 16384, 4096, 1, 0, 45),    # every 8-column segment in two groups
    (16, 8192, 17, 1, 9, 46),
])
def test_jagged_rowwise_ragged(rows, cols, G, mult, tail, seed):
    bits = adversarial((rows, cols), 100 + seed)
    offs = random_offsets(cols, G, seed, multiple=mult, short_tail=tail)
    check_rowwise(bits, offs)


def _pileup_offsets(cols):
    """Group ends for the many-groups rowwise kernel's per-element group
    words: 13, 14, 15 and 16 groups ending inside one 8-column segment (empty
    groups piled on one column and one-column groups), a segment with two
    boundaries that also holds the last group's end (elements past it belong
    to no group), and random groups of about 16 columns elsewhere."""
    ends = []
    base = 1000
    for k in (13, 14, 15, 16):
        start = base + 3                                   # inside the segment [base, base + 8)
        ends += [start] * (k - 4) + [start + 1, start + 2, start + 3, start + 4]
        base += 64
    g = np.random.default_rng(77)
    ends += list(np.sort(g.integers(base + 8, cols - 40, size=600)))
    last = (cols - 40) // 8 * 8
    ends += [last + 2, last + 5]                           # two ends in one segment, then no group
    return np.maximum.accumulate(np.array(sorted(ends), dtype=np.int64)).astype(np.int32)


@pytest.mark.parametrize("rows,cols,seed", [(8, 16384, 47), (700, 16384, 48), (6, 16381, 49),
                                            (5, 8191, 50)])
def test_jagged_rowwise_boundary_pileups(rows, cols, seed):
    bits = adversarial((rows, cols), 100 + seed)
    offs = _pileup_offsets(cols)
    assert offs.size > 16 and offs[-1] < cols
    check_rowwise(bits, offs)


@pytest.mark.parametrize("G,cols,tail,seed", [(1024, 16384, 1, 51), (256, 16384, 2, 52),
                                               (2000, 16384, 3, 53), (300, 16381, 0, 54)])
def test_jagged_rowwise_random_narrow_groups(G, cols, tail, seed):
    """Random group ends (about 16, 64, 8 and 55 columns per group) over the
    full register window: segments with one, two and more boundaries; the
    last case's last group covers the row's partial last segment."""
    bits = adversarial((12, cols), 100 + seed)
    offs = random_offsets(cols, G, seed, short_tail=tail)
    check_rowwise(bits, offs)


def test_jagged_rowwise_empty_extent_writes_empty_group_scales():
    bits = np.zeros((4, 0), dtype=np.uint16)
    x = torch.zeros((4, 8), dtype=torch.bfloat16, device="cuda")[:, :0]
    q, s = jagged_rowwise(x, i32_dev([0, 0, 0]))
    assert np.all(s.view(np.uint32) == 0x57CBBA10)
    _, os_ = oracle.quantize_jagged_rowwise(bits, np.array([0, 0, 0], dtype=np.int32))
    assert_same_bytes(s, os_, "scales")


@pytest.mark.parametrize("rows,cols,G,mult,tail,seed", [
    (1000, 64, 4, 1, 0, 11),
    (4099, 40, 7, 1, 3, 12),
    (20000, 8, 8, 16, 0, 13),
    (3000, 96, 1, 1, 0, 14),
    (5000, 16, 64, 1, 9, 15),      # G <= 64: largest-group-first order
    (7000, 24, 100, 1, 0, 16),     # G > 64: identity order
    (17, 264, 5, 1, 0, 17),
    (33, 8, 3, 1, 1, 18),
    (4100, 16, 1, 1, 0, 19),       # one group longer than the register window
    (9300, 24, 1, 1, 7, 20),       # ring: several passes, ragged ends
    (13000, 72, 2, 1, 0, 21),
    (2049, 40, 2, 1, 0, 22),
    (3000, 64, 1, 1, 0, 23),
    (6100, 136, 3, 1, 5, 24),
    (16384, 64, 64, 256, 0, 25),   # short groups packed, waves inside one group
    (5000, 40, 200, 1, 0, 26),     # packs of up to 64 groups, waves across groups
    (3000, 16, 1000, 1, 3, 27),    # groups of a few rows, many per lane
    (20000, 24, 30, 16, 0, 28),    # long and short groups interleaved
    (4096, 8, 4096, 1, 0, 29),     # the most groups, most of them empty
    (20000, 40, 65, 1, 3, 34),     # G just past 64: the one-group-per-thread table
    (40000, 24, 100, 16, 0, 31),   # long and short groups mixed, the same table
    (9000, 16, 512, 1, 5, 32),     # G = the workgroup's threads
    (9000, 16, 513, 1, 0, 33),     # one past: the chunked table
])
def test_jagged_colwise_ragged(rows, cols, G, mult, tail, seed):
    bits = adversarial((rows, cols), 200 + seed)
    offs = random_offsets(rows, G, seed, multiple=mult, short_tail=tail)
    check_colwise(bits, offs)


def test_jagged_colwise_empty_extent():
    x = torch.zeros((16, 16), dtype=torch.bfloat16, device="cuda")[:0]
    q, s = jagged_colwise(x, i32_dev([0, 0]))
    assert np.all(s.view(np.uint32) == 0x57CBBA10)


def test_rowwise_on_transposed_view_matches_row_major():
    """grad_out^T given as a transposed view of a row-major tensor."""
    rows, cols = 96, 3000
    bits = adversarial((rows, cols), 31)
    offs = random_offsets(cols, 6, 31, short_tail=5)
    base = bf16_dev(np.ascontiguousarray(bits.T))         # (cols, rows) row-major
    view = base.t()                                        # (rows, cols), strides (1, rows)
    assert view.stride() == (1, rows)
    q, s = jagged_rowwise(view, i32_dev(offs))
    oq, os_ = oracle.quantize_jagged_rowwise(bits, offs, canary=CANARY)
    assert_same_bytes(q, oq, "rowwise (transposed view) q")
    assert_same_bytes(s, os_, "rowwise (transposed view) scales")


@pytest.mark.parametrize("rows,cols,ends", [
    (40, 7000, [17, 3100, 3100, 6999]),     # groups split into chunks, an empty group, a tail
    (24, 20000, [3, 19999]),                # a long group starting off 16 columns
    (16, 4608, [1536, 1537, 3073, 4608]),   # ends at and past chunk multiples
])
def test_rowwise_on_transposed_view_long_groups(rows, cols, ends):
    """The transposed view with groups longer than a chunk: their chunks
    exchange maxima through the scale slots."""
    bits = adversarial((rows, cols), 33 + cols % 97)
    offs = np.array(ends, np.int32)
    view = bf16_dev(np.ascontiguousarray(bits.T)).t()
    q, s = jagged_rowwise(view, i32_dev(offs))
    oq, os_ = oracle.quantize_jagged_rowwise(bits, offs, canary=CANARY)
    assert_same_bytes(q, oq, f"rowwise (transposed view) q {ends}")
    assert_same_bytes(s, os_, f"rowwise (transposed view) scales {ends}")


def test_colwise_on_column_major_input():
    rows, cols = 2500, 48
    bits = adversarial((rows, cols), 41)
    offs = random_offsets(rows, 5, 41, short_tail=4)
    base = bf16_dev(np.ascontiguousarray(bits.T))         # (cols, rows) row-major
    view = base.t()                                        # (rows, cols) column-major
    q, s = jagged_colwise(view, i32_dev(offs))
    oq, os_ = oracle.quantize_jagged_colwise(bits, offs, canary=CANARY)
    assert_same_bytes(q, oq, "colwise (column-major in) q")
    assert_same_bytes(s, os_, "colwise (column-major in) scales")


def test_side_stream_and_determinism():
    a, offs = workloads.small_rowwise()
    x, o = bf16_dev(a), i32_dev(offs)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        q1, s1 = jagged_rowwise(x, o, stream=side)
    q2, s2 = jagged_rowwise(x, o)
    assert np.array_equal(q1, q2) and np.array_equal(s1.view(np.uint32), s2.view(np.uint32))


# ---------------------------------------------------------------------- MX

@pytest.mark.parametrize("mode", ["floor", "rceil"])
@pytest.mark.parametrize("E,N,K,seed", [(1, 128, 256, 1), (3, 96, 200, 2), (2, 512, 1032, 3)])
def test_mx_3d_colwise(E, N, K, seed, mode):
    w = np.stack([adversarial((N, K), 300 + seed * 10 + e) for e in range(E)])
    w[0, 0:32, 3] = 0                                           # zero block
    w[-1, 32:64, 5] = 0x8000                                    # negative zeros
    w[-1, N - 32:N, 7] = (np.arange(32, dtype=np.uint16) * 3) & 0x7F   # subnormal block
    w[0, 0:32, 9] = workloads.to_bf16_bits(
        np.random.default_rng(seed).standard_normal(32).astype(np.float32) * np.float32(2.0 ** 100))
    q, s = mx_3d_colwise(bf16_dev(w), mode=mode)
    oq, os_ = oracle.quantize_mx_3d_colwise(w, mode=mode)
    assert_same_bytes(q, oq, "mx 3d q")
    assert_same_bytes(s, os_, "mx 3d scales")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("E,N,K", [(2731, 160, 520), (8200, 32, 264)])
def test_mx_3d_colwise_many_tiles(E, N, K):
    """Grids of more than 16384 tiles, which the kernel walks in XCD chunks of
    column-tile pairs: an odd last column tile (3 tiles of 256, 256 and 8
    columns; 2 of 256 and 8), a ragged last row tile (160 = 128 + 32 rows)
    or a single one (32 rows), and grids that are not a whole number of
    8-chunk rounds (16386 and 16400 tiles), against the oracle on every
    expert."""
    w = workloads.normal_bf16((E, N, K), 11 + N)
    w[0, 0:32, 3] = 0                                           # zero block
    w[E - 1, N - 32:N, K - 1] = 0x8000                          # negative zeros, last column
    q, s = mx_3d_colwise(bf16_dev(w))
    oq, os_ = oracle_pool.split_op("quantize_mx_3d_colwise", w, align=1)
    assert_same_bytes(q, oq, "mx 3d many tiles q")
    assert_same_bytes(s, os_, "mx 3d many tiles scales")


@pytest.mark.parametrize("mode", ["floor", "rceil"])
def test_mx_3d_sweep_pattern_small(mode):
    w = np.stack([workloads.mx3d_sweep_expert(e, N=256, K=512) for e in range(2)])
    q, s = mx_3d_colwise(bf16_dev(w), mode=mode)
    oq, os_ = oracle.quantize_mx_3d_colwise(w, mode=mode)
    assert_same_bytes(q, oq, "mx 3d sweep q")
    assert_same_bytes(s, os_, "mx 3d sweep scales")
    assert (s == 0).sum() > 0


@pytest.mark.parametrize("mode", ["floor", "rceil"])
@pytest.mark.parametrize("rows,cols,seed", [(64, 256, 1), (5, 96, 2), (300, 4096, 3)])
def test_mx_rowwise(rows, cols, seed, mode):
    x = adversarial((rows, cols), 400 + seed)
    x[0, :32] = 0
    x[-1, 32:64] = np.arange(32, dtype=np.uint16) + 1
    q, s = mx_rowwise(bf16_dev(x), mode=mode)
    oq, os_ = oracle.quantize_mx_rowwise(x, mode=mode)
    assert_same_bytes(q, oq, "mx rowwise q")
    assert_same_bytes(s, os_, "mx rowwise scales")


# --------------------------------------------------------------- blockwise

@pytest.mark.parametrize("br,bc,rows,cols", [
    (1, 128, 3, 128), (1, 128, 256, 512), (1, 128, 77, 1152),
    (128, 128, 128, 128), (128, 128, 256, 384), (128, 128, 384, 1024),
    (128, 1, 128, 8), (128, 1, 256, 328),
])
def test_blockwise(br, bc, rows, cols):
    x = adversarial((rows, cols), 500 + rows + cols + br)
    x[:br, :bc] = 0                                             # zero block
    q, s = blockwise(bf16_dev(x), br, bc)
    oq, os_ = oracle.quantize_blockwise(x, br, bc)
    assert_same_bytes(q, oq, f"blockwise {br}x{bc} q")
    assert_same_bytes(s, os_, f"blockwise {br}x{bc} scales")


@pytest.mark.parametrize("qlayout", ["row", "col"])
@pytest.mark.parametrize("view", ["row_major", "transposed"])
@pytest.mark.parametrize("br,bc,rows,cols", [
    (1, 128, 16, 128), (1, 128, 272, 640), (1, 128, 400, 1152),
    (128, 128, 128, 128), (128, 128, 384, 640),
    (128, 1, 128, 16), (128, 1, 256, 328),
])
def test_blockwise_every_layout(br, bc, rows, cols, view, qlayout):
    """Every block shape with x row-major or a transposed view of a
    row-major tensor, into row-major or column-major q: the layouts the
    blockwise backward's transposed operands need, read in place."""
    x = adversarial((rows, cols), 900 + rows + cols + br)
    x[:br, :bc] = 0                                             # zero block
    if view == "row_major":
        dx = bf16_dev(x)
    else:
        dx = bf16_dev(np.ascontiguousarray(x.T)).t()          # x as a transposed view
        assert dx.stride(0) == 1
    if view == "transposed" and qlayout == "row" and (br, bc) == (128, 1) and cols % 16:
        # 1 x 128 blocks of the underlying tensor into its column-major q:
        # the tile kernel takes that tensor's rows (these columns) in 16s
        blockwise(dx, br, bc, qlayout=qlayout, expect=1)
        return
    q, s = blockwise(dx, br, bc, qlayout=qlayout)
    oq, os_ = oracle.quantize_blockwise(x, br, bc)
    what = f"blockwise {br}x{bc} {view} -> {qlayout}-major"
    assert_same_bytes(q, oq, what + " q")
    assert_same_bytes(s, os_, what + " scales")


def test_no_nan_codes_anywhere():
    x = adversarial((256, 1024), 9)
    for br, bc in ((1, 128), (128, 128)):
        q, _ = blockwise(bf16_dev(x), br, bc)
        assert not np.any((q & 0x7F) == 0x7F)


@pytest.mark.parametrize("mode", ["floor", "rceil"])
def test_mx_every_bf16_amax(mode):
    """One 32-element block per positive finite bf16 value v, holding v and
    31 smaller values: every e8m0 code each mode can produce, with the
    rceil threshold mantissas 96 / 97 and the clamp at code 0."""
    v = np.arange(0x7F80, dtype=np.uint16)              # 0 .. largest finite
    n = v.size
    g = np.random.default_rng(5)
    frac = g.integers(0, 0x7F80, size=(n, 31)).astype(np.uint16)
    frac = np.minimum(frac, v[:, None]) | (g.integers(0, 2, size=(n, 31)).astype(np.uint16) << 15)
    x = np.ascontiguousarray(np.concatenate([v[:, None], frac], axis=1).reshape(n // 32, 1024))
    q, s = mx_rowwise(bf16_dev(x), mode=mode)
    oq, os_ = oracle.quantize_mx_rowwise(x, mode=mode)
    assert_same_bytes(q, oq, f"mx rowwise {mode} q (every amax)")
    assert_same_bytes(s, os_, f"mx rowwise {mode} scales (every amax)")


def test_jagged_colwise_row_stride_past_2_23():
    """A row stride past 2^23 elements (128 rows of x span more than 2^31
    bytes): one 3150-row group (four tiles, one streamed and read again)
    and a short group after it."""
    rows, cols, ldx = 3200, 16, (1 << 23) + 64
    bits = adversarial((rows, cols), 240)
    offs = np.array([3150, 3200], dtype=np.int32)
    buf = torch.empty((rows - 1) * ldx + cols, dtype=torch.bfloat16, device="cuda")
    view = buf.as_strided((rows, cols), (ldx, 1))
    view.copy_(bf16_dev(bits))
    q, s = jagged_colwise(view, i32_dev(offs))
    del view, buf
    torch.cuda.empty_cache()
    oq, os_ = oracle.quantize_jagged_colwise(bits, offs, canary=CANARY)
    assert_same_bytes(q, oq, "colwise (row stride 2^23 + 64) q")
    assert_same_bytes(s, os_, "colwise (row stride 2^23 + 64) scales")


def test_jagged_colwise_many_equal_groups():
    """64 groups of 256 rows (many experts, few tokens each): whole waves
    inside one group, four groups per 1024-row block."""
    bits = adversarial((16384, 72), 230)
    offs = np.arange(256, 16385, 256, dtype=np.int32)
    check_colwise(bits, offs)


@pytest.mark.parametrize("shift,pad", [(0, 0), (16, 0), (0, 16), (48, 32)])
def test_column_major_stores_on_and_off_the_lines(shift, pad):
    """The block kernel takes nontemporal stores only when q, its column
    stride and its batch stride sit on 128-byte lines, plain stores
    otherwise; both give the oracle's bytes (MX 3D colwise and blockwise
    128x1), and nothing outside the tensor is written."""
    E, N, K = 2, 256, 264
    w = adversarial((E, N, K), 950 + shift + pad)
    ldq = N + pad
    buf = torch.full((E * K * ldq + shift + 64,), CANARY, dtype=torch.uint8, device="cuda")
    s = torch.full((E * (N // 32) * K,), CANARY, dtype=torch.uint8, device="cuda")
    dw = bf16_dev(w)
    code = mxq.mxq_quantize_mx_3d_colwise(dw.data_ptr(), E, N, K, dw.stride(0), dw.stride(1),
                                          dw.stride(2), buf.data_ptr() + shift, K * ldq, 1, ldq,
                                          s.data_ptr(), (N // 32) * K, K, 1, 0,
                                          torch.cuda.current_stream().cuda_stream)
    assert code == 0
    torch.cuda.synchronize()
    raw = buf.cpu().numpy()
    q = np.lib.stride_tricks.as_strided(raw[shift:], (E, N, K), (K * ldq, 1, ldq))
    oq, os_ = oracle.quantize_mx_3d_colwise(w)
    assert_same_bytes(np.ascontiguousarray(q), oq, f"mx3d q (shift {shift}, pad {pad})")
    assert_same_bytes(s.cpu().numpy().reshape(E, N // 32, K), os_, "mx3d scales")
    assert np.all(raw[:shift] == CANARY) and np.all(raw[shift + E * K * ldq:] == CANARY)
    if pad:
        assert np.all(np.lib.stride_tricks.as_strided(raw[shift + N:], (E * K, pad), (ldq, 1)) == CANARY)

    rows, cols = 256, 200
    x = adversarial((rows, cols), 960 + shift + pad)
    ldq = rows + pad
    buf = torch.full((cols * ldq + shift + 64,), CANARY, dtype=torch.uint8, device="cuda")
    sc = torch.full((rows // 128 * cols,), float("nan"), dtype=torch.float32, device="cuda")
    dx = bf16_dev(x)
    code = mxq.mxq_quantize_blockwise(dx.data_ptr(), rows, cols, dx.stride(0), dx.stride(1), 128, 1,
                                      buf.data_ptr() + shift, 1, ldq, sc.data_ptr(), cols, 1,
                                      torch.cuda.current_stream().cuda_stream)
    assert code == 0
    torch.cuda.synchronize()
    raw = buf.cpu().numpy()
    q = np.lib.stride_tricks.as_strided(raw[shift:], (rows, cols), (1, ldq))
    oq, os_ = oracle.quantize_blockwise(x, 128, 1)
    assert_same_bytes(np.ascontiguousarray(q), oq, f"blockwise 128x1 q (shift {shift}, pad {pad})")
    assert_same_bytes(sc.cpu().numpy().reshape(rows // 128, cols), os_, "blockwise 128x1 scales")
    assert np.all(raw[:shift] == CANARY) and np.all(raw[shift + cols * ldq:] == CANARY)
