"""GPU parity of the jagged MXFP8 entry points against the CPU oracle, byte
for byte: 32-element blocks restarting at every group start, with group
starts on and off 8/16/32-element boundaries, empty groups, offsets that stop
short of the extent (bytes past the last group and scale entries past the
last block keep the canary), one group, many groups, both scale modes, the
transposed-view and column-major layouts, and the full MoE backward shapes."""
import numpy as np
import pytest
import torch

import oracle
import oracle_pool
import workloads
from gpu_helpers import (CANARY, adversarial, assert_same_bytes, bf16_dev, i32_dev,
                         jagged_mx_colwise, jagged_mx_rowwise, random_offsets)

pytestmark = pytest.mark.gpu


def check_rowwise(bits, offs, mode):
    q, s = jagged_mx_rowwise(bf16_dev(bits), i32_dev(offs), mode)
    oq, os_ = oracle.quantize_jagged_mx_rowwise(bits, offs, mode=mode, canary=CANARY)
    assert_same_bytes(q, oq, f"jagged mx rowwise {mode} q")
    assert_same_bytes(s, os_, f"jagged mx rowwise {mode} scales")


def check_colwise(bits, offs, mode):
    q, s = jagged_mx_colwise(bf16_dev(bits), i32_dev(offs), mode)
    oq, os_ = oracle.quantize_jagged_mx_colwise(bits, offs, mode=mode, canary=CANARY)
    assert_same_bytes(q, oq, f"jagged mx colwise {mode} q")
    assert_same_bytes(s, os_, f"jagged mx colwise {mode} scales")


@pytest.mark.parametrize("mode", ["floor", "rceil"])
@pytest.mark.parametrize("rows,cols,G,mult,tail,seed", [
    (5, 1000, 4, 1, 0, 1),         # starts anywhere: element-wise pieces
    (17, 4096, 8, 8, 0, 2),        # starts on 8: 16-byte pieces, short last blocks
    (33, 3000, 6, 16, 8, 3),
    (16, 2048, 5, 32, 0, 4),       # blocks of every group full
    (3, 77, 1, 1, 0, 5),           # one group, ragged extent
    (4, 5000, 300, 1, 7, 6),       # many groups
    (2, 40, 64, 1, 0, 7),          # more groups than blocks
    (40, 1, 2, 1, 0, 8),
    (3, 9000, 4096, 1, 0, 9),      # the most groups, most of them empty
])
def test_jagged_mx_rowwise_ragged(rows, cols, G, mult, tail, seed, mode):
    bits = adversarial((rows, cols), 600 + seed)
    offs = random_offsets(cols, G, seed, multiple=mult, short_tail=tail)
    check_rowwise(bits, offs, mode)


@pytest.mark.parametrize("mode", ["floor", "rceil"])
@pytest.mark.parametrize("rows,cols,G,mult,tail,seed", [
    (1000, 64, 4, 1, 0, 11),       # starts anywhere: byte stores
    (4099, 40, 7, 16, 3, 12),      # starts on 16: 16-byte column pieces
    (2048, 264, 5, 32, 0, 13),
    (3000, 8, 1, 1, 0, 14),
    (5000, 16, 100, 1, 9, 15),     # many groups
    (33, 8, 3, 1, 1, 16),
    (300, 512, 2, 8, 0, 17),
    (9000, 16, 4096, 1, 0, 18),    # the most groups, most of them empty
])
def test_jagged_mx_colwise_ragged(rows, cols, G, mult, tail, seed, mode):
    bits = adversarial((rows, cols), 700 + seed)
    offs = random_offsets(rows, G, seed, multiple=mult, short_tail=tail)
    check_colwise(bits, offs, mode)


def test_jagged_mx_every_bf16_amax():
    """Every positive finite bf16 value leads one block (the rest of the
    block below it), with groups of 32 so every block is full: all codes of
    both modes on the device path."""
    v = np.arange(0x7F80, dtype=np.uint16)
    n = v.size
    g = np.random.default_rng(9)
    frac = np.minimum(g.integers(0, 0x7F80, size=(n, 31)).astype(np.uint16), v[:, None])
    x = np.ascontiguousarray(np.concatenate([v[:, None], frac], axis=1).reshape(n // 32, 1024))
    offs = np.arange(1, 33, dtype=np.int32) * 32
    for mode in ("floor", "rceil"):
        check_rowwise(x, offs, mode)


def test_jagged_mx_rowwise_transposed_view():
    rows, cols = 96, 3000
    bits = adversarial((rows, cols), 31)
    offs = random_offsets(cols, 6, 31, multiple=16, short_tail=5)
    base = bf16_dev(np.ascontiguousarray(bits.T))         # (cols, rows) row-major
    q, s = jagged_mx_rowwise(base.t(), i32_dev(offs))
    oq, os_ = oracle.quantize_jagged_mx_rowwise(bits, offs, canary=CANARY)
    assert_same_bytes(q, oq, "jagged mx rowwise (transposed view) q")
    assert_same_bytes(s, os_, "jagged mx rowwise (transposed view) scales")


def test_jagged_mx_colwise_column_major_input():
    rows, cols = 2500, 48
    bits = adversarial((rows, cols), 41)
    offs = random_offsets(rows, 5, 41, short_tail=4)
    base = bf16_dev(np.ascontiguousarray(bits.T))
    q, s = jagged_mx_colwise(base.t(), i32_dev(offs))
    oq, os_ = oracle.quantize_jagged_mx_colwise(bits, offs, canary=CANARY)
    assert_same_bytes(q, oq, "jagged mx colwise (column-major in) q")
    assert_same_bytes(s, os_, "jagged mx colwise (column-major in) scales")


def test_jagged_mx_empty_extents():
    x = torch.zeros((4, 8), dtype=torch.bfloat16, device="cuda")[:, :0]
    q, s = jagged_mx_rowwise(x, i32_dev([0, 0]))
    assert np.all(s == CANARY)
    x = torch.zeros((16, 16), dtype=torch.bfloat16, device="cuda")[:0]
    q, s = jagged_mx_colwise(x, i32_dev([0, 0, 0]))
    assert np.all(s == CANARY)


@pytest.mark.parametrize("mode", ["floor", "rceil"])
def test_moe_bwd_grad_out_t_rowwise(mode):
    """grad_out^T (4096, 16384) with the 8 MoE token groups, every byte and
    scale against the oracle (run over row blocks in parallel); every row
    writes exactly sum ceil(n_g/32) scale entries."""
    go = workloads.moe_grad_out_t()
    offs = workloads.moe_offsets()
    q, s = jagged_mx_rowwise(bf16_dev(go), i32_dev(offs), mode)
    oq, os_ = oracle_pool.split_op("quantize_jagged_mx_rowwise", go, offs, mode=mode, canary=CANARY)
    assert_same_bytes(q, oq, f"moe grad_out^T jagged mx {mode} q")
    assert_same_bytes(s, os_, f"moe grad_out^T jagged mx {mode} scales")
    sizes = np.diff(np.concatenate([[0], offs]))
    nb = int(sum((n + 31) // 32 for n in sizes))
    assert np.all(s[:, nb:] == CANARY)
    assert not np.any((q & 0x7F) == 0x7F)


@pytest.mark.parametrize("mode", ["floor", "rceil"])
def test_moe_bwd_x_colwise(mode):
    x = workloads.moe_x()
    offs = workloads.moe_offsets()
    q, s = jagged_mx_colwise(bf16_dev(x), i32_dev(offs), mode)
    oq, os_ = oracle_pool.split_op("quantize_jagged_mx_colwise", x, offs, mode=mode, canary=CANARY)
    assert_same_bytes(q, oq, f"moe x jagged mx {mode} q")
    assert_same_bytes(s, os_, f"moe x jagged mx {mode} scales")
    sizes = np.diff(np.concatenate([[0], offs]))
    nb = int(sum((n + 31) // 32 for n in sizes))
    assert np.all(s[nb:] == CANARY)
    assert not np.any((q & 0x7F) == 0x7F)


@pytest.mark.parametrize("mode", ["floor", "rceil"])
def test_moe_bwd_unaligned_starts(mode):
    """Both MoE operands with the group ends moved by a few tokens, so group
    starts sit off 8- and 16-element boundaries (the bench's unaligned MX
    workload): every byte against the oracle."""
    offs = workloads.moe_offsets_unaligned()
    assert np.any(offs[:-1] % 16 != 0)
    go = workloads.moe_grad_out_t()
    q, s = jagged_mx_rowwise(bf16_dev(go), i32_dev(offs), mode)
    oq, os_ = oracle_pool.split_op("quantize_jagged_mx_rowwise", go, offs, mode=mode, canary=CANARY)
    assert_same_bytes(q, oq, f"unaligned grad_out^T jagged mx {mode} q")
    assert_same_bytes(s, os_, f"unaligned grad_out^T jagged mx {mode} scales")
    del go, q, s, oq, os_
    x = workloads.moe_x()
    q, s = jagged_mx_colwise(bf16_dev(x), i32_dev(offs), mode)
    oq, os_ = oracle_pool.split_op("quantize_jagged_mx_colwise", x, offs, mode=mode, canary=CANARY)
    assert_same_bytes(q, oq, f"unaligned x jagged mx {mode} q")
    assert_same_bytes(s, os_, f"unaligned x jagged mx {mode} scales")
