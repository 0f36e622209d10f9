"""GPU parity of the jagged colwise call with a workspace (long token groups
cut into chunks that exchange their column maxima through the workspace)
against the oracle, byte for byte (the tile kernel up to 65,265 rows, the
split kernel beyond): the MoE backward operand at full size,
one group of every row, groups just past chunk and tile multiples, starts off
16-row boundaries, empty groups, rows past the last group, many groups, a
column count off the strip width; the waiting chunks' fallback (forced from
the host with a negative or zero wait bound); the workspace left zero-filled
after every call; repeated calls and graph replays on one workspace; and the
argument errors."""
import numpy as np
import pytest
import torch

import mxfp8_quantization_moe_amd as mxq
import oracle
import oracle_pool
import workloads
from gpu_helpers import (CANARY, DEV, adversarial, assert_same_bytes, bf16_dev, colwise_workspace,
                         i32_dev, jagged_colwise_ws, random_offsets)

pytestmark = pytest.mark.gpu


def check(bits, offs, spin=None, what=""):
    rows, cols = bits.shape
    ws = colwise_workspace(rows, cols, len(offs))
    q, s = jagged_colwise_ws(bf16_dev(bits), i32_dev(offs), ws, spin=spin)
    if bits.size > (1 << 22):
        oq, os_ = oracle_pool.split_op("quantize_jagged_colwise", bits, offs, canary=CANARY)
    else:
        oq, os_ = oracle.quantize_jagged_colwise(bits, offs, canary=CANARY)
    assert_same_bytes(q, oq, f"colwise ws q {what}")
    assert_same_bytes(s, os_, f"colwise ws scales {what}")
    assert int(torch.count_nonzero(ws)) == 0, "workspace not left zero-filled"


def test_moe_backward_operand():
    check(workloads.moe_x(), workloads.moe_offsets(), what="moe")


@pytest.mark.parametrize("rows,cols,ends,seed", [
    (16384, 256, [16384], 1),                       # one group (the split kernel): 6 chunks per strip
    (12000, 192, [6145, 12000], 2),                 # two groups just past 2 chunks
    (9300, 64, [3072, 3073, 6145, 9216, 9300], 3),  # at and past chunk multiples
    (7000, 136, [17, 3100, 3100, 6999], 4),         # starts off 16, an empty group, a tail
    (5000, 72, [1025, 2050, 4100, 5000], 5),        # just past one tile
    (20000, 8, [3, 19999], 6),                      # a tiny group, a long one off 16
    (6000, 64, [1536, 1537, 3073, 4608, 4609, 6000], 7),   # at and past 1536-row chunks
    (3000, 200, [499, 998, 1011, 1523, 3000], 8),   # just past a 512-row tile, off 16
    (3000, 264, [256, 257, 513, 640, 768, 769, 3000], 9),   # at and past 256-row chunks and 128-row tiles
    (2000, 520, [5, 261, 777, 2000], 10),           # chunks and tiles of groups starting off 16 rows
    (16384, 264, [0, 0, 0, 16384], 11),             # the tile kernel: 64 chunks per column tile
])
def test_long_groups(rows, cols, ends, seed):
    check(adversarial((rows, cols), 3000 + seed), np.array(ends, np.int32), what=str(ends))


@pytest.mark.parametrize("spin", [-1, 0])
def test_waiting_fallback(spin):
    """A negative bound never waits (every chunk of a split group reduces the
    group's rows itself); zero looks once."""
    bits = adversarial((13000, 264), 3100)
    check(bits, np.array([100, 6600, 6600, 13000], np.int32), spin=spin, what=f"spin {spin}")


@pytest.mark.parametrize("rows,cols,G,mult,tail,seed", [
    (16384, 512, 8, 16, 0, 11), (10000, 200, 64, 1, 7, 12), (40000, 16, 300, 1, 0, 13),
    (30000, 8, 4096, 1, 3, 14), (4096, 4096, 3, 16, 0, 15),
    # the one-group-per-thread table (up to 256 groups with 4-wave workgroups), and one past it
    (20000, 24, 65, 1, 0, 16), (30000, 16, 200, 16, 5, 17), (12000, 8, 256, 1, 0, 18),
    (12000, 8, 257, 1, 0, 19),
])
def test_random_groups(rows, cols, G, mult, tail, seed):
    offs = random_offsets(rows, G, seed, multiple=mult, short_tail=tail)
    check(adversarial((rows, cols), 3200 + seed), offs, what=f"G={G}")


@pytest.mark.parametrize("rows,ends", [
    (32625, [15] * 255 + [32625]),    # 255 one-tile chunks of 128 rows from row 0 (short groups on average)
    (32626, [15] * 255 + [32626]),    # one row more: two-tile chunks
    (65265, [15] * 15 + [65265]),     # the tile kernel's limit: 255 chunks of 256 rows
    (65266, [15] * 15 + [65266]),     # past it: the split kernel with the workspace
    (70000, [100, 69000, 70000]),     # long groups: the split kernel
])
def test_kernel_limits(rows, ends):
    check(adversarial((rows, 72), 3300 + rows % 7), np.array(ends, np.int32), what=f"{rows} rows")


def test_repeated_calls_and_smaller_second_call():
    """One workspace for several calls in a row, the later ones on fewer rows."""
    bits = adversarial((12288, 128), 3300)
    offs = np.array([7000, 12288], np.int32)
    ws = colwise_workspace(12288, 128, 2)
    x = bf16_dev(bits)
    d_offs = i32_dev(offs)
    oq, os_ = oracle.quantize_jagged_colwise(bits, offs, canary=CANARY)
    for _ in range(3):
        q, s = jagged_colwise_ws(x, d_offs, ws)
        assert_same_bytes(q, oq, "repeat q")
        assert_same_bytes(s, os_, "repeat scales")
    small = np.array([4000, 7000], np.int32)
    q, s = jagged_colwise_ws(bf16_dev(bits[:7000]), i32_dev(small), ws)
    oq, os_ = oracle.quantize_jagged_colwise(bits[:7000], small, canary=CANARY)
    assert_same_bytes(q, oq, "smaller q")
    assert_same_bytes(s, os_, "smaller scales")
    assert int(torch.count_nonzero(ws)) == 0


def test_graph_replays():
    """Captured once, replayed several times with new input between replays:
    the workspace is left clean by each replay."""
    rows, cols = 9000, 128
    offs = np.array([500, 8000, 9000], np.int32)
    a = adversarial((rows, cols), 3400)
    b = adversarial((rows, cols), 3401)
    x = bf16_dev(a)
    d_offs = i32_dev(offs)
    ws = colwise_workspace(rows, cols, 3)
    ldq = 9008
    q = torch.empty(cols * ldq, dtype=torch.uint8, device=DEV)
    s = torch.empty(3 * cols, dtype=torch.float32, device=DEV)
    stream = torch.cuda.Stream()
    nbytes = ws.numel() * 4

    def call():
        code = mxq.mxq_quantize_jagged_colwise_ws(
            x.data_ptr(), rows, cols, cols, 1, d_offs.data_ptr(), 3, q.data_ptr(), 1, ldq, s.data_ptr(),
            cols, 1, ws.data_ptr(), nbytes, torch.cuda.current_stream().cuda_stream)
        assert code == 0

    with torch.cuda.stream(stream):
        call()                       # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        call()
    for k, bits in enumerate([a, b, a, b]):
        x.copy_(bf16_dev(bits))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        oq, os_ = oracle.quantize_jagged_colwise(bits, offs)
        got_q = q.as_strided((rows, cols), (1, ldq)).cpu().numpy()
        assert_same_bytes(got_q, oq, f"replay {k} q")
        assert_same_bytes(s.view(3, cols).cpu().numpy(), os_, f"replay {k} scales")
        assert int(torch.count_nonzero(ws)) == 0


def test_column_major_input_needs_no_workspace():
    bits = adversarial((3000, 40), 3500)
    offs = np.array([0, 1500, 3000], np.int32)
    base = bf16_dev(np.ascontiguousarray(bits.T)).t()          # column-major x
    ws = torch.zeros(1, dtype=torch.int32, device=DEV)
    q, s = jagged_colwise_ws(base, i32_dev(offs), ws, ws_bytes=0)
    oq, os_ = oracle.quantize_jagged_colwise(bits, offs, canary=CANARY)
    assert_same_bytes(q, oq, "column-major in q")
    assert_same_bytes(s, os_, "column-major in scales")


def test_argument_errors():
    x = bf16_dev(adversarial((4096, 64), 3600))
    offs = i32_dev([4096])
    need = mxq.mxq_jagged_colwise_workspace_bytes(4096, 64, 1)
    assert need > 0
    ws = colwise_workspace(4096, 64, 1)
    jagged_colwise_ws(x, offs, ws, ws_bytes=need - 4, expect=mxq.MXQ_ERR_WORKSPACE)
    code = mxq.mxq_quantize_jagged_colwise_ws(x.data_ptr(), 4096, 64, 64, 1, offs.data_ptr(), 1,
                                              ws.data_ptr(), 1, 4096, ws.data_ptr(), 64, 1, 0, need, 0)
    assert code == mxq.MXQ_ERR_WORKSPACE                         # no workspace
    assert int(torch.count_nonzero(ws)) == 0


def test_tensor_binding_with_workspace():
    bits = workloads.moe_x()[:4096]
    offs = np.array([100, 3000, 4096], np.int32)
    x = bf16_dev(bits)
    ws = mxq.jagged_colwise_workspace(4096, 4096, 3)
    q, s = mxq.quantize_jagged_colwise(x, i32_dev(offs), workspace=ws)
    q2, s2 = mxq.quantize_jagged_colwise(x, i32_dev(offs))
    assert torch.equal(q.view(torch.uint8), q2.view(torch.uint8)) and torch.equal(s, s2)
