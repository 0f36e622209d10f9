"""Pins of the oracle's quantization ops.

The second implementation here is written with torch CPU tensor expressions
(masked amax, float32 division and product, clamp, the library's float8 cast),
mirroring the "pure PyTorch implementation" the jagged-scaling pages test
their kernels against.  It shares no code with ``oracle.c``.  On top of that:
brute force over every composition of a tiny extent into groups, the G = 1
special case (plain per-row scaling), the closed-form invariants (the amax
element maps to +-448, or to the top binade of e4m3 under MX floor scaling),
group locality, and the exact 2^k shift of MX codes.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

EPS = float(np.float32(1e-12))


# ----------------------------------------------------- torch-expression twin

def _f32(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(workloads.bf16_bits_to_f32(np.ascontiguousarray(bits)).copy())


def _cast(y: torch.Tensor) -> np.ndarray:
    return y.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def twin_jagged_rowwise(x_bits, offs, canary=0):
    x = _f32(x_bits)
    rows, cols = x.shape
    q = np.full((rows, cols), canary, dtype=np.uint8)
    s = np.zeros((rows, len(offs)), dtype=np.float32)
    col = torch.arange(cols)
    lo = 0
    for g, hi in enumerate(int(o) for o in offs):
        mask = (col >= lo) & (col < hi)
        amax = torch.where(mask[None, :], x.abs(), torch.zeros(())).amax(dim=1)
        sc = torch.tensor(448.0, dtype=torch.float32) / amax.clamp_min(EPS)
        s[:, g] = sc.numpy()
        qq = _cast(x * sc[:, None])
        q[:, mask.numpy()] = qq[:, mask.numpy()]
        lo = hi
    return q, s


def twin_jagged_colwise(x_bits, offs, canary=0):
    qT, sT = twin_jagged_rowwise(np.ascontiguousarray(x_bits.T), offs, canary)
    return np.ascontiguousarray(qT.T), np.ascontiguousarray(sT.T)


def twin_blockwise(x_bits, br, bc):
    x = _f32(x_bits)
    rows, cols = x.shape
    xb = x.reshape(rows // br, br, cols // bc, bc)
    amax = xb.abs().amax(dim=(1, 3))
    sc = torch.tensor(448.0, dtype=torch.float32) / amax.clamp_min(EPS)
    q = _cast(xb * sc[:, None, :, None]).reshape(rows, cols)
    return q, sc.numpy()


def _mx_exponent(amax: torch.Tensor) -> torch.Tensor:
    """OCP MX shared exponent for E4M3 (emax = 8), floor rounding, clamped to
    the e8m0 range, via the library's frexp."""
    _, e = torch.frexp(amax.double())
    se = (e.to(torch.int64) - 1) - 8
    se = torch.where(amax == 0, torch.full_like(se, -127), se)
    return se.clamp(-127, 127)


def _mx_exponent_rceil(amax: torch.Tensor) -> torch.Tensor:
    """rceil reading: ceil(log2(amax / 448)), via frexp of the float64 quotient
    (an exact power of two has mantissa 0.5 and is its own ceiling); the
    quotient of a bf16 by 448 = 7 * 64 is never within a rounding error of a
    power of two unless it equals one."""
    m, e = torch.frexp(amax.double() / 448.0)
    se = torch.where(m == 0.5, e.to(torch.int64) - 1, e.to(torch.int64))
    se = torch.where(amax == 0, torch.full_like(se, -127), se)
    return se.clamp(-127, 127)


def twin_mx_blocks(x_bits, block_axis_len, reshape_fn, unshape_fn, mode="floor"):
    x = _f32(x_bits)
    xb = reshape_fn(x)                       # (..., 32) with the block on the last axis
    amax = xb.abs().amax(dim=-1)
    se = _mx_exponent(amax) if mode == "floor" else _mx_exponent_rceil(amax)
    mult = torch.ldexp(torch.ones_like(amax, dtype=torch.float64), -se).to(torch.float32)
    q = _cast(xb * mult[..., None])
    return unshape_fn(q), (se + 127).to(torch.uint8).numpy()


def twin_mx_rowwise(x_bits, mode="floor"):
    rows, cols = x_bits.shape
    return twin_mx_blocks(x_bits, 32, lambda x: x.reshape(rows, cols // 32, 32),
                          lambda q: q.reshape(rows, cols), mode)


def twin_mx_3d(w_bits, mode="floor"):
    E, N, K = w_bits.shape

    def shape(w):
        return w.reshape(E, N // 32, 32, K).permute(0, 1, 3, 2)   # (E, NB, K, 32)

    def unshape(q):
        return np.ascontiguousarray(q.transpose(0, 1, 3, 2).reshape(E, N, K))

    return twin_mx_blocks(w_bits, 32, shape, unshape, mode)


# ------------------------------------------------------------------ inputs

def adversarial_bf16(shape, seed):
    """N(0,1) bf16 with signed zeros, subnormals, huge values and exact ties."""
    g = np.random.default_rng(seed)
    v = g.standard_normal(size=shape).astype(np.float32)
    bits = workloads.to_bf16_bits(v)
    flat = bits.reshape(-1)
    n = flat.size
    pick = g.choice(n, size=max(1, n // 8), replace=False)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F,
                         0x3F80, 0xBF80, 0x43E0, 0x3C00], dtype=np.uint16)
    flat[pick] = specials[g.integers(specials.size, size=pick.size)]
    return bits


def compositions(n, parts):
    """All ways to write n as an ordered sum of ``parts`` non-negative ints."""
    for cuts in itertools.combinations_with_replacement(range(n + 1), parts - 1):
        edges = (0,) + cuts + (n,)
        yield [edges[i + 1] - edges[i] for i in range(parts)]


# ------------------------------------------------------------------- jagged

@pytest.mark.parametrize("G", [1, 2, 3, 4])
def test_jagged_rowwise_all_compositions(G):
    extent = 12 if G == 4 else 20
    x = workloads.normal_bf16((3, extent), 11 + G)
    x[0, ::5] = 0x8000                        # negative zeros
    n = 0
    for sizes in compositions(extent, G):
        offs = np.cumsum(sizes).astype(np.int32)
        q, s = oracle.quantize_jagged_rowwise(x, offs, canary=0xA5)
        tq, ts = twin_jagged_rowwise(x, offs, canary=0xA5)
        assert np.array_equal(q, tq), sizes
        assert np.array_equal(s.view(np.uint32), ts.view(np.uint32)), sizes
        n += 1
    assert n == math.comb(extent + G - 1, G - 1)


@pytest.mark.parametrize("G", [2, 3])
def test_jagged_colwise_all_compositions_and_short_tail(G):
    extent = 18
    x = workloads.normal_bf16((extent, 5), 21 + G)
    for sizes in compositions(extent, G):
        for tail in (0, 3):                   # offs[-1] < extent leaves a tail in no group
            if tail and sizes[-1] < tail:
                continue
            sz = list(sizes)
            sz[-1] -= tail
            offs = np.cumsum(sz).astype(np.int32)
            q, s = oracle.quantize_jagged_colwise(x, offs, canary=0xA5)
            tq, ts = twin_jagged_colwise(x, offs, canary=0xA5)
            assert np.array_equal(q, tq), (sz, tail)
            assert np.array_equal(s.view(np.uint32), ts.view(np.uint32)), (sz, tail)
            if tail:
                assert np.all(q[extent - tail:] == 0xA5)


def test_jagged_small_workloads_match_twin():
    a, offs = workloads.small_rowwise()
    q, s = oracle.quantize_jagged_rowwise(a, offs)
    tq, ts = twin_jagged_rowwise(a, offs)
    assert np.array_equal(q, tq) and np.array_equal(s.view(np.uint32), ts.view(np.uint32))
    b, offs_b = workloads.small_colwise()
    q, s = oracle.quantize_jagged_colwise(b, offs_b)
    tq, ts = twin_jagged_colwise(b, offs_b)
    assert np.array_equal(q, tq) and np.array_equal(s.view(np.uint32), ts.view(np.uint32))
    # exactly one empty group, and its scale is 448 / fp32(1e-12)
    sizes = np.diff(np.concatenate([[0], offs]))
    assert (sizes == 0).sum() == 1
    g0 = int(np.nonzero(sizes == 0)[0][0])
    oq, os_ = oracle.quantize_jagged_rowwise(a, offs)
    assert np.all(os_[:, g0].view(np.uint32) == 0x57CBBA10)


def test_jagged_adversarial_values_match_twin():
    x = adversarial_bf16((16, 96), 5)
    offs = np.array([0, 7, 40, 41, 96], dtype=np.int32)
    q, s = oracle.quantize_jagged_rowwise(x, offs)
    tq, ts = twin_jagged_rowwise(x, offs)
    assert np.array_equal(q, tq) and np.array_equal(s.view(np.uint32), ts.view(np.uint32))


def test_single_group_is_per_row_scaling():
    x = workloads.normal_bf16((8, 64), 3)
    q, s = oracle.quantize_jagged_rowwise(x, np.array([64], dtype=np.int32))
    xf = _f32(x)
    amax = xf.abs().amax(dim=1, keepdim=True).clamp_min(EPS)
    ref = _cast(xf * (torch.tensor(448.0) / amax))
    assert np.array_equal(q, ref)


def test_amax_element_maps_to_448_for_every_bf16_amax():
    """For every finite bf16 amax >= 1e-12 the element holding it encodes to
    +-448 (0x7E / 0xFE) under the fp32 multiplier."""
    bits = np.arange(0x8000, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]
    amax = workloads.bf16_bits_to_f32(bits)
    bits = bits[amax >= EPS]
    rows = bits.size
    x = np.zeros((rows, 128), dtype=np.uint16)
    x[:, 0] = bits
    x[1::2, 0] |= 0x8000                      # negative amax element on odd rows
    x[:, 1] = bits >> 1                       # a smaller companion value
    q, _ = oracle.quantize_blockwise(x, 1, 128)
    assert np.all(q[0::2, 0] == 0x7E)
    assert np.all(q[1::2, 0] == 0xFE)
    assert rows == 21491


def test_group_locality():
    x = workloads.normal_bf16((6, 80), 9)
    offs = np.array([16, 16, 48, 80], dtype=np.int32)
    q, s = oracle.quantize_jagged_rowwise(x, offs)
    y = x.copy()
    y[:, 20:30] = workloads.normal_bf16((6, 10), 10)      # perturb group 2 only
    q2, s2 = oracle.quantize_jagged_rowwise(y, offs)
    keep = np.r_[0:16, 48:80]
    assert np.array_equal(q[:, keep], q2[:, keep])
    assert np.array_equal(s[:, [0, 1, 3]], s2[:, [0, 1, 3]])
    # moving one boundary changes only the two adjacent groups
    offs3 = np.array([16, 16, 40, 80], dtype=np.int32)
    q3, s3 = oracle.quantize_jagged_rowwise(x, offs3)
    assert np.array_equal(q[:, 0:16], q3[:, 0:16])
    assert np.array_equal(s[:, [0, 1]], s3[:, [0, 1]])


# ---------------------------------------------------------------- blockwise

@pytest.mark.parametrize("br,bc", [(1, 128), (128, 128), (128, 1), (1, 32), (32, 32)])
def test_blockwise_matches_twin(br, bc):
    x = adversarial_bf16((256, 256), 100 + br + bc)
    q, s = oracle.quantize_blockwise(x, br, bc)
    tq, ts = twin_blockwise(x, br, bc)
    assert np.array_equal(q, tq)
    assert np.array_equal(s.view(np.uint32), ts.view(np.uint32))
    assert not np.any((q & 0x7F) == 0x7F)


def test_blockwise_zero_block():
    x = workloads.normal_bf16((128, 256), 4)
    x[:, :128] = 0
    x[5, 7] = 0x8000
    q, s = oracle.quantize_blockwise(x, 128, 128)
    assert s.view(np.uint32)[0, 0] == 0x57CBBA10
    assert np.all(q[:, :128][x[:, :128] == 0] == 0)
    assert q[5, 7] == 0x80


# ----------------------------------------------------------------------- MX

def test_mx_rowwise_matches_twin():
    x = adversarial_bf16((64, 256), 31)
    x[3, :32] = 0                             # zero block
    x[4, 32:64] = np.arange(32, dtype=np.uint16) + 1      # subnormal block
    q, s = oracle.quantize_mx_rowwise(x)
    tq, ts = twin_mx_rowwise(x)
    assert np.array_equal(q, tq) and np.array_equal(s, ts)
    assert s[3, 0] == 0 and np.all(q[3, :32] == 0)
    assert s[4, 1] == 0 and np.any(q[4, 32:64] != 0)      # 2^127 multiplier revives subnormals


def test_mx_3d_matches_twin_with_special_blocks():
    E, N, K = 2, 96, 40
    w = np.stack([adversarial_bf16((N, K), 41 + e) for e in range(E)])
    w[0, 0:32, 3] = 0
    w[1, 32:64, 5] = 0x8000
    w[1, 64:96, 7] = (np.arange(32, dtype=np.uint16) * 3) & 0x7F   # subnormals
    q, s = oracle.quantize_mx_3d_colwise(w)
    tq, ts = twin_mx_3d(w)
    assert np.array_equal(q, tq) and np.array_equal(s, ts)
    assert s[0, 0, 3] == 0 and s[1, 1, 5] == 0
    assert np.all(q[1, 32:64, 5] == 0x80)


def test_mx_amax_element_in_top_binade():
    w = workloads.mx3d_sweep_expert(0, N=256, K=64)[None]
    q, s = oracle.quantize_mx_3d_colwise(w)
    E, N, K = w.shape
    mag = w & 0x7FFF
    blk = mag.reshape(E, N // 32, 32, K)
    arg = blk.argmax(axis=2)
    qb = q.reshape(E, N // 32, 32, K)
    top = np.take_along_axis(qb, arg[:, :, None, :], axis=2)[:, :, 0, :] & 0x7F
    nz = s > 0
    assert np.all((top[nz] >= 0x78) & (top[nz] <= 0x7E))
    assert np.all(top[~nz] == 0)              # zero blocks of the sweep
    assert (~nz).sum() > 0


def test_mx_power_of_two_shift():
    x = workloads.normal_bf16((8, 64), 77)
    q, s = oracle.quantize_mx_rowwise(x)
    for k in (-20, -3, 5, 20):
        f = workloads.bf16_bits_to_f32(x) * np.float32(2.0 ** k)
        y = workloads.to_bf16_bits(f)          # exact: power-of-two scaling
        q2, s2 = oracle.quantize_mx_rowwise(y)
        assert np.array_equal(q, q2)
        assert np.array_equal(s2.astype(int), s.astype(int) + k)


def test_mx_rceil_matches_twin():
    x = adversarial_bf16((64, 256), 32)
    x[3, :32] = 0
    x[4, 32:64] = np.arange(32, dtype=np.uint16) + 1
    q, s = oracle.quantize_mx_rowwise(x, mode="rceil")
    tq, ts = twin_mx_rowwise(x, mode="rceil")
    assert np.array_equal(q, tq) and np.array_equal(s, ts)
    w = np.stack([adversarial_bf16((96, 40), 51 + e) for e in range(2)])
    w[0, 0:32, 3] = 0
    q3, s3 = oracle.quantize_mx_3d_colwise(w, mode="rceil")
    tq3, ts3 = twin_mx_3d(w, mode="rceil")
    assert np.array_equal(q3, tq3) and np.array_equal(s3, ts3)


def test_mx_rceil_never_saturates_and_top_code_in_upper_half():
    """Under rceil every block's amax element lands in (224, 448] before the
    cast (e4m3 codes 0x76..0x7E); no element is clipped; floor and rceil agree
    on a block exactly when its amax mantissa is at most 1.75."""
    x = workloads.mx3d_sweep_expert(1, N=256, K=64)
    xr = np.ascontiguousarray(x.T)                       # (64, 256): 1x32 blocks along dim 1
    q, s = oracle.quantize_mx_rowwise(xr, mode="rceil")
    qf, sf = oracle.quantize_mx_rowwise(xr)
    v = workloads.bf16_bits_to_f32(xr).astype(np.float64).reshape(64, 8, 32)
    se = s.astype(np.int64) - 127
    scaled = np.abs(v) * np.ldexp(1.0, -se)[..., None]   # exact in float64
    assert np.all(scaled <= 448.0)
    top = (q.reshape(64, 8, 32) & 0x7F).max(axis=2)
    nz = np.abs(v).max(axis=2) > 0
    assert np.all((top[nz] >= 0x76) & (top[nz] <= 0x7E))
    mant = (xr.reshape(64, 8, 32) & 0x7FFF).max(axis=2) & 0x7F
    same = s == sf
    assert np.array_equal(same[nz], (mant <= 96)[nz])
    assert np.array_equal(q.reshape(64, 8, 32)[same], qf.reshape(64, 8, 32)[same])


# ---------------------------------------------------------------- jagged MX

def twin_jagged_mx_rowwise(x_bits, offs, mode="floor", canary=0xA5):
    """Each group's columns, zero-padded on the right to a multiple of 32 (a
    zero changes no block amax), go through the MX twin above; the padding
    is dropped again and the groups' scale columns are concatenated."""
    rows, cols = x_bits.shape
    G = len(offs)
    nb = (cols + 31) // 32 + G - 1
    q = np.full((rows, cols), canary, dtype=np.uint8)
    s = np.full((rows, nb), canary, dtype=np.uint8)
    lo, b = 0, 0
    for hi in [int(v) for v in offs]:
        n = hi - lo
        if n > 0:
            pad = -n % 32
            seg = np.concatenate([x_bits[:, lo:hi], np.zeros((rows, pad), np.uint16)], axis=1)
            tq, ts = twin_mx_rowwise(seg, mode)
            q[:, lo:hi] = tq[:, :n]
            s[:, b:b + ts.shape[1]] = ts
            b += ts.shape[1]
        lo = hi
    return q, s


@pytest.mark.parametrize("mode", ["floor", "rceil"])
@pytest.mark.parametrize("G", [1, 2, 3])
def test_jagged_mx_rowwise_all_compositions(G, mode):
    extent = 70 if G < 3 else 40
    x = adversarial_bf16((3, extent), 61 + G)
    n = 0
    for sizes in compositions(extent, G):
        offs = np.cumsum(sizes).astype(np.int32)
        q, s = oracle.quantize_jagged_mx_rowwise(x, offs, mode=mode, canary=0xA5)
        tq, ts = twin_jagged_mx_rowwise(x, offs, mode)
        assert np.array_equal(q, tq), sizes
        assert np.array_equal(s, ts), sizes
        n += 1
    assert n == math.comb(extent + G - 1, G - 1)


def test_jagged_mx_short_tail_and_empty_groups_keep_canary():
    x = adversarial_bf16((4, 200), 71)
    offs = np.array([0, 33, 33, 97, 150], dtype=np.int32)       # tail 150..199 in no group
    q, s = oracle.quantize_jagged_mx_rowwise(x, offs, canary=0xA5)
    tq, ts = twin_jagged_mx_rowwise(x, offs)
    assert np.array_equal(q, tq) and np.array_equal(s, ts)
    assert np.all(q[:, 150:] == 0xA5)
    # blocks: 0 + 2 + 0 + 2 + 2 = 6 of a capacity of 7 + 5 - 1 = 11
    assert np.all(s[:, 6:] == 0xA5) and np.all(s[:, :6] != 0xA5)


@pytest.mark.parametrize("mode", ["floor", "rceil"])
def test_jagged_mx_aligned_groups_equal_plain_mx(mode):
    """With every group a multiple of 32 long, the blocks are the plain MX
    blocks and the scale columns are the plain ones in order."""
    x = adversarial_bf16((8, 512), 72)
    offs = np.array([64, 64, 224, 480, 512], dtype=np.int32)
    q, s = oracle.quantize_jagged_mx_rowwise(x, offs, mode=mode, canary=0xA5)
    pq, ps = oracle.quantize_mx_rowwise(x, mode=mode)
    assert np.array_equal(q, pq)
    assert np.array_equal(s[:, :16], ps) and np.all(s[:, 16:] == 0xA5)


@pytest.mark.parametrize("mode", ["floor", "rceil"])
def test_jagged_mx_colwise_is_rowwise_of_transpose(mode):
    x = adversarial_bf16((150, 6), 73)
    offs = np.array([17, 17, 80, 149], dtype=np.int32)
    q, s = oracle.quantize_jagged_mx_colwise(x, offs, mode=mode, canary=0xA5)
    tq, ts = twin_jagged_mx_rowwise(np.ascontiguousarray(x.T), offs, mode)
    assert np.array_equal(q, tq.T) and np.array_equal(s, ts.T)


def test_jagged_mx_group_locality():
    """Scaling one group by 2^k shifts only that group's scale codes by k and
    leaves every q byte unchanged."""
    x = workloads.normal_bf16((4, 160), 74)
    offs = np.array([45, 100, 160], dtype=np.int32)
    q, s = oracle.quantize_jagged_mx_rowwise(x, offs)
    y = x.copy()
    f = workloads.bf16_bits_to_f32(y[:, 45:100]) * np.float32(2.0 ** 7)
    y[:, 45:100] = workloads.to_bf16_bits(f)
    q2, s2 = oracle.quantize_jagged_mx_rowwise(y, offs)
    assert np.array_equal(q, q2)
    d = s2.astype(int) - s.astype(int)
    # group 0: blocks 0-1, group 1: blocks 2-3, group 2: blocks 4-5
    assert np.all(d[:, 2:4] == 7) and np.all(d[:, [0, 1, 4, 5]] == 0)
