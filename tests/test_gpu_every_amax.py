"""Every finite bf16 amax >= 1e-12 (21,491 values) through each
fp32-multiplier path on the GPU, against the oracle byte for byte: blockwise
1 x 128 and 128 x 128, jagged rowwise (with a group boundary inside a 16-byte
segment) and jagged colwise (a long group of more than one register tile and
a packed short group).

These paths convert without the +-448 clamp, so every product
RN32(amax * 448 / amax) that lands just above 448 (in (448, 448 + 2^-15])
must still come out as 448: each unit's amax element must encode to 0x7E or
0xFE.  The other elements of each unit are random values of magnitude at
most its amax, with random signs."""
import numpy as np
import pytest

import oracle_pool
import workloads
from gpu_helpers import (CANARY, assert_same_bytes, bf16_dev, blockwise, i32_dev, jagged_colwise,
                         jagged_rowwise)

pytestmark = pytest.mark.gpu

EPS = np.float32(1e-12)


def every_amax() -> np.ndarray:
    bits = np.arange(0x7F80, dtype=np.uint16)            # +0 .. largest finite
    return bits[workloads.bf16_bits_to_f32(bits) >= EPS]


def below(g, amax_bits: np.ndarray, shape) -> np.ndarray:
    """Random bf16 patterns with |value| <= the given amax (broadcast over
    ``shape``) and random signs."""
    mag = g.integers(0, amax_bits.astype(np.int64) + 1, size=shape).astype(np.uint16)
    return mag | (g.integers(0, 2, size=shape).astype(np.uint16) << 15)


def signed(amax_bits: np.ndarray, g) -> np.ndarray:
    return amax_bits | (g.integers(0, 2, size=amax_bits.shape).astype(np.uint16) << 15)


def check_amax_codes(q_vals: np.ndarray):
    assert np.all((q_vals & 0x7F) == 0x7E)


def test_count():
    assert every_amax().size == 21491


def test_blockwise_1x128_every_amax():
    A = every_amax()
    n = A.size
    g = np.random.default_rng(21)
    x = below(g, A[:, None], (n, 128))
    pos = g.integers(0, 128, size=n)
    x[np.arange(n), pos] = signed(A, g)
    q, s = blockwise(bf16_dev(x), 1, 128)
    oq, os_ = oracle_pool.split_op("quantize_blockwise", x, 1, 128)
    assert_same_bytes(q, oq, "1x128 every amax q")
    assert_same_bytes(s, os_, "1x128 every amax scales")
    check_amax_codes(q[np.arange(n), pos])


def test_blockwise_128x128_every_amax():
    """One 128 x 128 block per amax, laid side by side: (128, 128 * 21491);
    each block holds its amax element among values within three binades
    below it."""
    A = every_amax()
    n = A.size
    g = np.random.default_rng(22)
    lo = np.maximum(A.astype(np.int32) - 0x180, 0).astype(np.uint16)
    mag = lo[None, :, None] + g.integers(0, 0x181, size=(128, n, 128), dtype=np.uint16)
    np.minimum(mag, A[None, :, None], out=mag)
    mag |= g.integers(0, 2, size=mag.shape, dtype=np.uint16) << 15
    x = mag.reshape(128, 128 * n)
    rr = g.integers(0, 128, size=n)
    cc = g.integers(0, 128, size=n) + 128 * np.arange(n)
    x[rr, cc] = signed(A, g)
    q, s = blockwise(bf16_dev(x), 128, 128)
    oq, os_ = oracle_pool.split_op("quantize_blockwise", x, 128, 128, align=128, axis=1)
    assert_same_bytes(q, oq, "128x128 every amax q")
    assert_same_bytes(s, os_, "128x128 every amax scales")
    check_amax_codes(q[rr, cc])


def test_jagged_rowwise_every_amax():
    """(21491, 128) with groups [0, 61) and [61, 128): group 0 of row r has
    amax A[r], group 1 a permuted one; the boundary falls inside a 16-byte
    segment, so both the packed and the element-wise stores are used."""
    A = every_amax()
    n = A.size
    g = np.random.default_rng(23)
    A1 = A[g.permutation(n)]
    x = np.empty((n, 128), dtype=np.uint16)
    x[:, :61] = below(g, A[:, None], (n, 61))
    x[:, 61:] = below(g, A1[:, None], (n, 67))
    p0 = g.integers(0, 61, size=n)
    p1 = g.integers(61, 128, size=n)
    x[np.arange(n), p0] = signed(A, g)
    x[np.arange(n), p1] = signed(A1, g)
    offs = np.array([61, 128], dtype=np.int32)
    q, s = jagged_rowwise(bf16_dev(x), i32_dev(offs))
    oq, os_ = oracle_pool.split_op("quantize_jagged_rowwise", x, offs, canary=CANARY)
    assert_same_bytes(q, oq, "jagged rowwise every amax q")
    assert_same_bytes(s, os_, "jagged rowwise every amax scales")
    check_amax_codes(q[np.arange(n), p0])
    check_amax_codes(q[np.arange(n), p1])


def test_jagged_colwise_every_amax():
    """(2048, 21496) with groups [0, 1200) (longer than a register tile) and
    [1200, 2048) (a packed short group): group 0 of column c has amax A[c],
    group 1 a permuted one (the last 5 columns repeat the first amax)."""
    A = every_amax()
    n = A.size
    cols = (n + 7) // 8 * 8
    g = np.random.default_rng(24)
    A0 = np.concatenate([A, A[: cols - n]])
    A1 = A0[g.permutation(cols)]
    x = np.empty((2048, cols), dtype=np.uint16)
    x[:1200] = below(g, A0[None, :], (1200, cols))
    x[1200:] = below(g, A1[None, :], (848, cols))
    p0 = g.integers(0, 1200, size=cols)
    p1 = g.integers(1200, 2048, size=cols)
    x[p0, np.arange(cols)] = signed(A0, g)
    x[p1, np.arange(cols)] = signed(A1, g)
    offs = np.array([1200, 2048], dtype=np.int32)
    q, s = jagged_colwise(bf16_dev(x), i32_dev(offs))
    oq, os_ = oracle_pool.split_op("quantize_jagged_colwise", x, offs, canary=CANARY)
    assert_same_bytes(q, oq, "jagged colwise every amax q")
    assert_same_bytes(s, os_, "jagged colwise every amax scales")
    check_amax_codes(q[p0, np.arange(cols)])
    check_amax_codes(q[p1, np.arange(cols)])
