"""GPU parity of the jagged colwise call WITHOUT a workspace on long token
groups: chunks of one long group exchange their column maxima through the
group's own fp32 scale slots (cleared by a small kernel first), so no row is
read twice.  Up to 65,265 rows the call runs the tile kernel (chunks of 128
or 256 rows x 256 columns, at most 255 per group); longer extents run the split
kernel (chunks of 1536 rows x 64 columns, at most 255 per group).  Byte for
byte against the oracle: one group of every row, groups at and past chunk
multiples, starts off 16-row boundaries, empty groups, rows past the last
group, up to 256 groups, the most chunks a group may have in either kernel
and one row more (the split kernel, resp. the path that reads long groups
twice, then takes the call), scale strides other than row-major, the
waiting chunks' fallback (forced from the host), scale buffers holding the
previous call's scales, and graph replays."""
import numpy as np
import pytest
import torch

import mxfp8_quantization_moe_amd as mxq
import oracle
import oracle_pool
import workloads
from gpu_helpers import (CANARY, DEV, _gather_f32, _gather_u8, adversarial, assert_same_bytes,
                         bf16_dev, f32_canary, i32_dev, jagged_colwise, random_offsets, round16,
                         stream_handle, u8_canary)

pytestmark = pytest.mark.gpu

CHUNK = 1536            # rows per chunk of the split kernel (3 tiles of 512 rows)
TILE_CHUNK = 256        # rows per chunk of the tile kernel (2 tiles of 128 rows)
MAX_CHUNKS = 255        # chunks a group may have when the scale slots carry the counts


def want(bits, offs):
    if bits.size > (1 << 22):
        return oracle_pool.split_op("quantize_jagged_colwise", bits, offs, canary=CANARY)
    return oracle.quantize_jagged_colwise(bits, offs, canary=CANARY)


def call(x, offs, scale_layout="gc", spin=None, q=None, s=None):
    """Column-major q (padded column stride); scales (G, cols) row-major
    ("gc"), column-major ("cg"), or row-major with a padded row stride
    ("gc_pad").  ``spin``: the test-only entry with that wait bound and no
    workspace.  Returns (q, scales) gathered into logical order."""
    rows, cols = x.shape
    G = offs.numel()
    ldq = round16(max(rows, 1))
    if scale_layout == "gc":
        ss, n = (cols, 1), G * cols
    elif scale_layout == "cg":
        ss, n = (1, G), G * cols
    else:
        ss, n = (cols + 24, 1), G * (cols + 24)
    q = u8_canary(cols * ldq) if q is None else q
    s = f32_canary(n) if s is None else s
    args = (x.data_ptr(), rows, cols, x.stride(0), x.stride(1), offs.data_ptr(), G, q.data_ptr(), 1,
            ldq, s.data_ptr(), ss[0], ss[1])
    if spin is None:
        code = mxq.mxq_quantize_jagged_colwise(*args, stream_handle())
    else:
        code = mxq.mxq_debug_jagged_colwise_ws_spin(*args, 0, 0, spin, stream_handle())
    assert code == 0, code
    torch.cuda.synchronize()
    return _gather_u8(q, (rows, cols), (1, ldq)), _gather_f32(s, (G, cols), ss), q, s


def check(bits, offs, what="", **kw):
    q, s, _, _ = call(bf16_dev(bits), i32_dev(offs), **kw)
    oq, os_ = want(bits, offs)
    assert_same_bytes(q, oq, f"colwise q {what}")
    assert_same_bytes(s, os_, f"colwise scales {what}")


def test_moe_backward_operand():
    check(workloads.moe_x(), workloads.moe_offsets(), what="moe")


@pytest.mark.parametrize("rows,cols,ends,seed", [
    (16384, 256, [16384], 1),                       # one group (the split kernel): 11 chunks per strip
    (12000, 192, [6145, 12000], 2),
    (9300, 64, [3072, 3073, 6145, 9216, 9300], 3),
    (7000, 136, [17, 3100, 3100, 6999], 4),         # starts off 16, an empty group, a tail
    (20000, 8, [3, 19999], 6),                      # a tiny group, a long one off 16
    (6000, 64, [1536, 1537, 3073, 4608, 4609, 6000], 7),   # at and past chunk multiples
    (3000, 200, [499, 998, 1011, 1523, 3000], 8),
    (3000, 264, [256, 257, 513, 640, 768, 769, 3000], 9),   # at and past 256-row chunks and 128-row tiles
    (2000, 520, [5, 261, 777, 2000], 10),           # chunks and tiles of groups starting off 16 rows
    (16384, 264, [0, 0, 0, 16384], 11),             # the tile kernel: 64 chunks per column tile
])
def test_long_groups(rows, cols, ends, seed):
    check(adversarial((rows, cols), 5000 + seed), np.array(ends, np.int32), what=str(ends))


@pytest.mark.parametrize("layout", ["cg", "gc_pad"])
def test_scale_strides(layout):
    """Scale slots addressed column-major and with a padded row stride."""
    bits = adversarial((9000, 72), 5100)
    check(bits, np.array([2000, 8000, 9000], np.int32), what=layout, scale_layout=layout)


@pytest.mark.parametrize("spin", [-1, 0])
def test_waiting_fallback(spin):
    """A negative bound never waits (every chunk reduces its group's rows
    itself and the last one out still writes the scale); zero looks once."""
    bits = adversarial((13000, 264), 5200)
    check(bits, np.array([100, 6600, 6600, 13000], np.int32), what=f"spin {spin}", spin=spin)


@pytest.mark.parametrize("rows,cols,G,mult,tail,seed", [
    (16384, 512, 8, 16, 0, 11), (10000, 200, 64, 1, 7, 12), (30000, 16, 200, 16, 5, 17),
    (12000, 8, 256, 1, 0, 18), (12000, 8, 257, 1, 0, 19),   # 257: the path without chunks
])
def test_random_groups(rows, cols, G, mult, tail, seed):
    offs = random_offsets(rows, G, seed, multiple=mult, short_tail=tail)
    check(adversarial((rows, cols), 5300 + seed), offs, what=f"G={G}")


@pytest.mark.parametrize("extra", [0, 1])
def test_most_chunks(extra):
    """255 chunks of 1536 rows in one group (the counts' limit), and one row
    more, where the call reads the group twice instead."""
    rows = MAX_CHUNKS * CHUNK + extra
    bits = adversarial((rows, 8), 5400 + extra)
    check(bits, np.array([rows], np.int32), what=f"{rows} rows")


@pytest.mark.parametrize("extra", [0, 1])
def test_tile_kernel_most_chunks(extra):
    """255 chunks of 256 rows in one group, the tile kernel's limit: a
    15-row group, 14 empty ones (which keep the average group within the
    tile kernel's) and the long group, starting at row 15 so that its chunks
    cover it from row 0; a second 256-column tile of 8 columns.  One row more
    and the call takes the split kernel instead."""
    rows = MAX_CHUNKS * TILE_CHUNK - 15 + extra
    bits = adversarial((rows, 264), 5450 + extra)
    check(bits, np.array([15] * 15 + [rows], np.int32), what=f"{rows} rows")


@pytest.mark.parametrize("extra", [0, 1])
def test_tile_kernel_one_tile_chunks_most(extra):
    """255 chunks of 128 rows in one group (a 15-row group and 254 empty ones
    before it: groups of at most 128 rows on average take one-tile chunks),
    and one row more, where the call takes two-tile chunks instead."""
    rows = MAX_CHUNKS * 128 - 15 + extra
    bits = adversarial((rows, 264), 5460 + extra)
    check(bits, np.array([15] * 255 + [rows], np.int32), what=f"{rows} rows")


def test_previous_scales_in_the_slots():
    """Calls in a row on the same output buffers, the second on other rows:
    the slots hold the first call's scales (and canary bytes elsewhere) when
    the second call starts."""
    a = adversarial((9000, 128), 5500)
    b = adversarial((9000, 128), 5501)
    offs = np.array([700, 8000, 9000], np.int32)
    d_offs = i32_dev(offs)
    q, s, qb, sb = call(bf16_dev(a), d_offs)
    for bits in (b, a, b):
        q, s, _, _ = call(bf16_dev(bits), d_offs, q=qb, s=sb)
        oq, os_ = oracle.quantize_jagged_colwise(bits, offs)
        assert_same_bytes(q, oq, "repeat q")
        assert_same_bytes(s, os_, "repeat scales")


def test_graph_replays():
    """The clear kernel and the split kernel captured once, replayed several
    times with new input between replays."""
    rows, cols = 9000, 128
    offs = np.array([500, 8000, 9000], np.int32)
    a = adversarial((rows, cols), 5600)
    b = adversarial((rows, cols), 5601)
    x = bf16_dev(a)
    d_offs = i32_dev(offs)
    ldq = 9008
    q = torch.empty(cols * ldq, dtype=torch.uint8, device=DEV)
    s = torch.empty(3 * cols, dtype=torch.float32, device=DEV)
    stream = torch.cuda.Stream()

    def launch():
        code = mxq.mxq_quantize_jagged_colwise(
            x.data_ptr(), rows, cols, cols, 1, d_offs.data_ptr(), 3, q.data_ptr(), 1, ldq, s.data_ptr(),
            cols, 1, torch.cuda.current_stream().cuda_stream)
        assert code == 0

    with torch.cuda.stream(stream):
        launch()                     # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        launch()
    for k, bits in enumerate([b, a, b, a]):
        x.copy_(bf16_dev(bits))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        oq, os_ = oracle.quantize_jagged_colwise(bits, offs)
        got_q = q.as_strided((rows, cols), (1, ldq)).cpu().numpy()
        assert_same_bytes(got_q, oq, f"replay {k} q")
        assert_same_bytes(s.view(3, cols).cpu().numpy(), os_, f"replay {k} scales")


def test_same_result_as_the_workspace_call():
    """The two split paths agree on a full-size operand (the oracle already
    pins both; this guards the q bytes past the last group too)."""
    x = bf16_dev(workloads.moe_x())
    offs = i32_dev(workloads.moe_offsets_unaligned())
    q1, s1 = jagged_colwise(x, offs)
    from gpu_helpers import colwise_workspace, jagged_colwise_ws
    q2, s2 = jagged_colwise_ws(x, offs, colwise_workspace(*x.shape, offs.numel()))
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)
