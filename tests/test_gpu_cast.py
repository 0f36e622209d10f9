"""The device fp32 -> E4M3FN conversions against the oracle's encoder.

The quantization kernels convert through three forms of the hardware's
round-to-nearest-even conversion (v_cvt_pk_fp8_f32):
  * one value at a time after a v_med3_f32 clamp to +-448 (element-wise
    stores at group edges), through ``mxq_debug_cast_e4m3``;
  * four values at a time after the clamp (the e8m0 paths, whose scaled
    values reach 512), through ``mxq_debug_cast4_e4m3`` with unclamped=0;
  * four values at a time without the clamp (the fp32-multiplier paths:
    jagged rowwise / colwise and blockwise), through ``mxq_debug_cast4_e4m3``
    with unclamped=1.  That form is only ever fed |y| <= 448 + 2^-15 (the
    product of an element and 448 / max(amax, eps) rounded to fp32), so it is
    checked on every fp32 value of both signs in [2^-13, 464), and on a dense
    sample below; outside that range it is not used.
The oracle runs in parallel host processes (``oracle_pool``)."""
import numpy as np
import pytest
import torch

import mxfp8_quantization_moe_amd as mxq
import oracle
import oracle_pool

pytestmark = pytest.mark.gpu

FORMS = ("cast1", "cast4_clamped", "cast4_unclamped")


def device_cast(y: np.ndarray, form: str) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).cuda()
    if form == "cast1":
        out = mxq.debug_cast_e4m3(t)
    else:
        out = mxq.debug_cast4_e4m3(t, unclamped=(form == "cast4_unclamped"))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def compare(y: np.ndarray, what: str, form: str = "cast1"):
    got = device_cast(y, form)
    want = oracle_pool.e4m3_encode(y) if y.size > (1 << 20) else oracle.e4m3_encode(y)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (what, form, bad.size,
                           [(float(y[i]), hex(y[i:i+1].view(np.uint32)[0]), hex(got[i]), hex(want[i]))
                            for i in bad[:8]])


@pytest.mark.parametrize("form", FORMS)
def test_cast_all_bf16(form):
    b = np.arange(1 << 16, dtype=np.uint32)
    b = b[((b >> 7) & 0xFF) != 0xFF]
    y = (b << 16).view(np.float32)
    if form == "cast4_unclamped":
        y = y[np.abs(y) < 464]
    compare(y, "bf16", form)


@pytest.mark.parametrize("form", FORMS)
def test_cast_tie_neighbourhoods(form):
    mags = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32).view(np.uint32).astype(np.int64)
    k = np.arange(-256, 257, dtype=np.int64)
    pats = (mids[:, None] + k[None, :]).ravel()
    pats = pats[pats >= 0].astype(np.uint32)
    y = pats.view(np.float32)
    compare(np.concatenate([y, -y]), "ties", form)


@pytest.mark.parametrize("form", ["cast1", "cast4_clamped"])
@pytest.mark.parametrize("binade", [-12, -11, -10, -9, -7, -6, -1, 0, 7, 8])
def test_cast_whole_binades_clamped(binade, form):
    """Every fp32 value in [2^b, 2^(b+1)), both signs (2^24 values)."""
    start = (binade + 127) << 23
    pats = np.arange(start, start + (1 << 23), dtype=np.uint32)
    y = pats.view(np.float32)
    compare(np.concatenate([y, -y]), f"binade {binade}", form)


@pytest.mark.parametrize("binade", list(range(-13, 9)))
def test_cast_unclamped_every_value_below_464(binade):
    """The form of the fp32-multiplier paths on every fp32 value of
    [2^b, 2^(b+1)) that is below 464, both signs: every binade from 2^-13
    (all results there are +-0 or the smallest subnormal codes) to the
    saturation boundary, the values the form is used on."""
    start = (binade + 127) << 23
    pats = np.arange(start, start + (1 << 23), dtype=np.uint32)
    y = pats.view(np.float32)
    y = y[y < 464.0]
    compare(np.concatenate([y, -y]), f"unclamped binade {binade}", "cast4_unclamped")


def test_cast_unclamped_below_2_pow_13_and_ragged_tail():
    """Below 2^-13 every value rounds to a signed zero: a dense sample of the
    range, fp32 subnormals included; an odd count exercises the short last
    quad."""
    pats = np.arange(0, (127 - 13) << 23, 331, dtype=np.uint32)
    y = pats.view(np.float32)
    edge = np.array([447.99997, 448.0, 448.00003, 463.99997], np.float32)
    y = np.concatenate([edge, -edge, y, -y])
    y = y[: (y.size - 3) // 4 * 4 + 3]
    assert y.size % 4 == 3
    compare(y, "below 2^-13", "cast4_unclamped")


@pytest.mark.parametrize("form", ["cast1", "cast4_clamped"])
def test_cast_saturation_and_specials(form):
    y = np.array([448.0, 448.00003, 463.99997, 464.0, 479.0, 480.0, 512.0, 1e6, 3.4e38,
                  0.0, -0.0, 1e-45, -1e-45, 1.2e-38, -1.2e-38, 2.0 ** -10, -(2.0 ** -10),
                  2.0 ** -10 * 1.0000001, 3 * 2.0 ** -10], dtype=np.float32)
    compare(np.concatenate([y, -y]), "specials", form)
    # fp32 subnormals and the tiny range, densely
    pats = np.arange(0, 1 << 23, 97, dtype=np.uint32)
    y = pats.view(np.float32)
    compare(np.concatenate([y, -y]), "fp32 subnormals", form)


@pytest.mark.parametrize("form", ["cast1", "cast4_clamped"])
def test_cast_random_fp32(form):
    g = np.random.default_rng(3)
    pats = g.integers(0, 0x7F800000, size=8_000_000, dtype=np.int64).astype(np.uint32)
    y = pats.view(np.float32)
    compare(np.concatenate([y, -y]), "random", form)
