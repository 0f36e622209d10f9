"""The device cast (v_med3_f32 saturation + v_cvt_pk_fp8_f32) against the
oracle's E4M3FN encoder, over whole binades of fp32 inputs, every bf16 value,
the neighbourhood of every rounding tie, and out-of-range values.  Every
quantized byte the kernels write comes out of this cast."""
import numpy as np
import pytest
import torch

import mxfp8_quantization_moe_amd as mxq
import oracle

pytestmark = pytest.mark.gpu


def device_cast(y: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).cuda()
    out = mxq.debug_cast_e4m3(t)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def compare(y: np.ndarray, what: str):
    got = device_cast(y)
    want = oracle.e4m3_encode(y)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (what, [(float(y[i]), hex(y[i:i+1].view(np.uint32)[0]), hex(got[i]),
                                   hex(want[i])) for i in bad[:8]])


def test_cast_all_bf16():
    b = np.arange(1 << 16, dtype=np.uint32)
    b = b[((b >> 7) & 0xFF) != 0xFF]
    compare((b << 16).view(np.float32), "bf16")


def test_cast_tie_neighbourhoods():
    mags = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32).view(np.uint32).astype(np.int64)
    k = np.arange(-256, 257, dtype=np.int64)
    pats = (mids[:, None] + k[None, :]).ravel()
    pats = pats[pats >= 0].astype(np.uint32)
    y = pats.view(np.float32)
    compare(np.concatenate([y, -y]), "ties")


@pytest.mark.parametrize("binade", [-12, -11, -10, -9, -7, -6, -1, 0, 7, 8])
def test_cast_whole_binades(binade):
    """Every fp32 value in [2^b, 2^(b+1)), both signs (2^24 values)."""
    start = (binade + 127) << 23
    pats = np.arange(start, start + (1 << 23), dtype=np.uint32)
    y = pats.view(np.float32)
    compare(np.concatenate([y, -y]), f"binade {binade}")


def test_cast_saturation_and_specials():
    y = np.array([448.0, 448.00003, 463.99997, 464.0, 479.0, 480.0, 512.0, 1e6, 3.4e38,
                  0.0, -0.0, 1e-45, -1e-45, 1.2e-38, -1.2e-38, 2.0 ** -10, -(2.0 ** -10),
                  2.0 ** -10 * 1.0000001, 3 * 2.0 ** -10], dtype=np.float32)
    compare(np.concatenate([y, -y]), "specials")
    # fp32 subnormals and the tiny range, densely
    pats = np.arange(0, 1 << 23, 97, dtype=np.uint32)
    y = pats.view(np.float32)
    compare(np.concatenate([y, -y]), "fp32 subnormals")


def test_cast_random_fp32():
    g = np.random.default_rng(3)
    pats = g.integers(0, 0x7F800000, size=8_000_000, dtype=np.int64).astype(np.uint32)
    y = pats.view(np.float32)
    compare(np.concatenate([y, -y]), "random")
