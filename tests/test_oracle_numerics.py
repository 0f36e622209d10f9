"""Pins of the oracle's scalar numerics against things other than itself.

* the OCP E4M3 fixed points (golden file, cited there);
* torch's CPU float32 -> float8_e4m3fn cast (a library routine that rounds to
  nearest-even but does not saturate; the reading adds saturation, so inputs
  are clamped to +-448 before the library cast);
* exact rational arithmetic (``fractions.Fraction``) with a hand-written
  correct rounding to binary32, for the fp32 quantize multiplier;
* the defining property of the MX "floor" shared exponent
  (amax / 2^se in [256, 512)) and its bit-field form, for the e8m0 code;
* the defining property of the "rceil" reading (amax / 2^se in (224, 448],
  the smallest non-saturating power of two), its mantissa-threshold form and
  closed forms at 448 * 2^k, for the rceil e8m0 code.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def torch_e4m3(y_f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(y_f32, dtype=np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def all_finite_bf16_bits() -> np.ndarray:
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (b >> 7) & 0xFF
    return b[exp != 0xFF]


def bits_to_f32(bits16: np.ndarray) -> np.ndarray:
    return (bits16.astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------ e4m3 encoder

def test_golden_ocp_points():
    rows = []
    with open(os.path.join(HERE, "golden", "ocp_e4m3_points.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                v, c = line.split()
                rows.append((float.fromhex(v), int(c, 16)))
    assert len(rows) >= 10
    for v, c in rows:
        assert oracle.e4m3_encode([v])[0] == c, (v, hex(c))
        assert oracle.e4m3_decode([c])[0] == v or (v == 0 and c in (0, 0x80))


def test_decode_matches_library_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ref[~nan], ours[~nan])
    # signed zero of code 0x80
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert codes.size == 254
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


def test_encoder_matches_library_on_all_bf16():
    bits = all_finite_bf16_bits()
    y = bits_to_f32(bits)
    assert np.array_equal(oracle.e4m3_encode(y), torch_e4m3(y))


def test_encoder_midpoints_and_neighbours():
    """Every midpoint between adjacent codes, and +-1..64 ulps around it:
    ties go to the even code, anything off the tie to the nearer code."""
    mags = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (mags[:-1] + mags[1:]) / 2)  # exact in fp32
    u = mids.view(np.uint32).astype(np.int64)
    k = np.arange(-64, 65, dtype=np.int64)
    pats = (u[:, None] + k[None, :]).ravel()
    pats = pats[pats >= 0].astype(np.uint32)
    y = pats.view(np.float32)
    y = np.concatenate([y, -y])
    ours = oracle.e4m3_encode(y)
    assert np.array_equal(ours, torch_e4m3(y))
    # the tie itself rounds to the even code
    tie_codes = oracle.e4m3_encode(mids)
    assert np.all(tie_codes % 2 == 0)


def test_encoder_random_fp32_and_saturation():
    g = np.random.default_rng(7)
    pats = g.integers(0, 0x43E00001, size=2_000_000, dtype=np.int64).astype(np.uint32)
    y = pats.view(np.float32)
    y = np.concatenate([y, -y])
    assert np.array_equal(oracle.e4m3_encode(y), torch_e4m3(y))
    big = np.array([448.0001, 463.9, 464.0, 480.0, 1e6, 3.0e38], dtype=np.float32)
    assert np.all(oracle.e4m3_encode(big) == 0x7E)
    assert np.all(oracle.e4m3_encode(-big) == 0xFE)


def test_encoder_tiny_values_keep_sign():
    tiny = np.array([2.0 ** -10, 2.0 ** -11, 1e-30, 1e-45], dtype=np.float32)
    assert np.all(oracle.e4m3_encode(tiny) == 0x00)
    assert np.all(oracle.e4m3_encode(-tiny) == 0x80)
    # 3 * 2^-10 is the tie between 2^-9 (0x01) and 2^-8 (0x02): even wins
    assert oracle.e4m3_encode([3 * 2.0 ** -10])[0] == 0x02


@pytest.mark.slow
def test_encoder_exhaustive_fp32_range():
    """All binary32 patterns with |y| <= 448 (about 2.3e9 values)."""
    top = 0x43E00000
    step = 1 << 24
    for start in range(0, top + 1, step):
        pats = np.arange(start, min(start + step, top + 1), dtype=np.uint32)
        y = pats.view(np.float32)
        assert np.array_equal(oracle.e4m3_encode(y), torch_e4m3(y)), hex(start)
        assert np.array_equal(oracle.e4m3_encode(-y), torch_e4m3(-y)), hex(start)


# ------------------------------------------------------- fp32 multiplier

def _round_fraction_to_fp32(q: Fraction) -> float:
    """Correct round-to-nearest-even of a positive rational to binary32
    (normal range only), by integer arithmetic."""
    assert q > 0
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    assert -126 <= e <= 127
    scaled = q / Fraction(2) ** (e - 23)          # in [2^23, 2^24)
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return float(Fraction(m) * Fraction(2) ** (e - 23))


def test_fp32_scale_exact_rational_all_bf16():
    bits = all_finite_bf16_bits()
    bits = bits[bits < 0x8000]                   # non-negative amax
    assert bits.size == 32640
    amax = bits_to_f32(bits)
    ours = oracle.fp32_scale(amax)
    eps = Fraction(float(np.float32(1e-12)))
    for a, s in zip(amax.tolist(), ours.tolist()):
        denom = max(Fraction(a), eps)
        assert s == _round_fraction_to_fp32(Fraction(448) / denom), a


def test_fp32_scale_closed_forms():
    for k in range(-39, 120):                    # 2^-39 > 1e-12: no clamp
        amax = np.float32(2.0 ** k)
        assert oracle.fp32_scale([amax])[0] == np.float32(448.0 * 2.0 ** -k)
    assert oracle.fp32_scale([448.0])[0] == 1.0
    assert oracle.fp32_scale([7.0])[0] == 64.0
    # empty group / zero block: 448 / fp32(1e-12)
    for a in (0.0, 1e-13, 2.0 ** -130):
        assert oracle.fp32_scale([a]).view(np.uint32)[0] == 0x57CBBA10


# ------------------------------------------------------------ e8m0 floor

def test_e8m0_defining_property_all_bf16():
    bits = all_finite_bf16_bits()
    bits = bits[bits < 0x8000]
    amax = bits_to_f32(bits)
    codes = oracle.e8m0_floor(amax).astype(np.int64)
    assert codes.min() == 0 and codes.max() == 246      # 255 (NaN) never occurs
    for a, c in zip(amax.tolist(), codes.tolist()):
        se = c - 127
        if a == 0.0:
            assert c == 0
            continue
        ratio = Fraction(a) / Fraction(2) ** se
        if c > 0:
            assert Fraction(256) <= ratio < Fraction(512), (a, c)
        else:
            # clamped at the minimum code: floor(log2 amax) - 8 <= -127
            assert ratio < Fraction(512)


def test_e8m0_matches_bit_field_form():
    """For normal bf16 amax the floor of log2 is the unbiased exponent field;
    below 2^-118 the code clamps to 0."""
    bits = all_finite_bf16_bits()
    bits = bits[bits < 0x8000]
    amax = bits_to_f32(bits)
    field = (bits.astype(np.int64) >> 7) & 0xFF
    expect = np.clip(field - 127 - 8, -127, 127) + 127
    assert np.array_equal(oracle.e8m0_floor(amax).astype(np.int64), expect)


def test_e8m0_power_of_two_closed_form():
    for k in range(-118, 128):
        assert oracle.e8m0_floor([np.float32(2.0 ** k)])[0] == k - 8 + 127


# ------------------------------------------------------------ e8m0 rceil

def test_e8m0_rceil_defining_property_all_bf16():
    """se is the smallest integer with amax <= 448 * 2^se: checked with exact
    rationals for every finite non-negative bf16 amax."""
    bits = all_finite_bf16_bits()
    bits = bits[bits < 0x8000]
    amax = bits_to_f32(bits)
    codes = oracle.e8m0_rceil(amax).astype(np.int64)
    assert codes.min() == 0 and codes.max() == 247
    for a, c in zip(amax.tolist(), codes.tolist()):
        se = c - 127
        if a == 0.0:
            assert c == 0
            continue
        ratio = Fraction(a) / Fraction(2) ** se
        assert ratio <= 448, (a, c)                  # never saturates
        if c > 0:
            assert ratio > 224, (a, c)               # se - 1 would saturate


def test_e8m0_rceil_mantissa_threshold_form():
    """448 = 1.75 * 2^8 and 1.75 is the 7-bit mantissa 96/128, so rceil
    exceeds floor by one exactly when the bf16 mantissa field is above 96."""
    bits = all_finite_bf16_bits()
    bits = bits[bits < 0x8000]
    amax = bits_to_f32(bits)
    field = (bits.astype(np.int64) >> 7) & 0xFF
    mant = bits.astype(np.int64) & 0x7F
    expect = np.clip(field - 135 + (mant > 96), -127, 127) + 127
    expect[amax == 0] = 0
    assert np.array_equal(oracle.e8m0_rceil(amax).astype(np.int64), expect)
    floor = oracle.e8m0_floor(amax).astype(np.int64)
    rceil = oracle.e8m0_rceil(amax).astype(np.int64)
    assert np.all((rceil - floor >= 0) & (rceil - floor <= 1))


def test_e8m0_rceil_closed_forms():
    for k in range(-126, 119):
        exact = np.float32(448.0 * 2.0 ** k)          # 1.75 * 2^(k+8): a bf16 value
        assert oracle.e8m0_rceil([exact])[0] == k + 127
        above = np.nextafter(exact, np.float32(np.inf))
        assert oracle.e8m0_rceil([above])[0] == k + 128
        assert oracle.e8m0_rceil([np.float32(2.0 ** (k + 8))])[0] == k + 127
    assert oracle.e8m0_rceil([np.float32(2.0 ** -149)])[0] == 0   # clamps at code 0
