"""GPU parity at the full workload sizes, in the launch configuration
bench.py times.  The GPU output of the whole tensor is compared byte for byte
with the oracle on sampled rows / columns / experts (the oracle computes those
one by one, each sample being a complete reduction unit), and whole-output
properties are checked at every size: no NaN codes, every scale of every
group or block equals the multiplier of that group's exact amax, and, for the
MX sweep, the expert-prefix property (running on W[:E] reproduces the first
E experts of the E=64 run)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import (CANARY, assert_same_bytes, bf16_dev, blockwise, i32_dev, jagged_colwise,
                         jagged_rowwise, mx_3d_colwise)

pytestmark = pytest.mark.gpu


def _fp32_scales_from_amax_bits(amax16: np.ndarray) -> np.ndarray:
    amax = workloads.bf16_bits_to_f32(amax16.astype(np.uint16))
    flat = np.unique(amax)
    table = dict(zip(flat.tolist(), oracle.fp32_scale(flat).tolist()))
    return np.vectorize(table.__getitem__, otypes=[np.float32])(amax)


def _no_nan_codes(q: np.ndarray):
    assert not np.any((q & 0x7F) == 0x7F)


def _sample(n, k, seed):
    g = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], g.choice(n, size=k, replace=False)]))


def test_moe_bwd_rowwise_grad_out_t():
    go = workloads.moe_grad_out_t()
    offs = workloads.moe_offsets()
    q, s = jagged_rowwise(bf16_dev(go), i32_dev(offs))
    rows = _sample(go.shape[0], 40, 1)
    oq, os_ = oracle.quantize_jagged_rowwise(go[rows], offs, canary=CANARY)
    assert_same_bytes(q[rows], oq, "moe_bwd rowwise q (sampled rows)")
    assert_same_bytes(s[rows], os_, "moe_bwd rowwise scales (sampled rows)")
    # every (row, group) scale is the multiplier of the group's exact amax
    mag = go & 0x7FFF
    lo = 0
    for g, hi in enumerate(offs.tolist()):
        amax = mag[:, lo:hi].max(axis=1) if hi > lo else np.zeros(go.shape[0], np.uint16)
        want = _fp32_scales_from_amax_bits(amax)
        assert_same_bytes(s[:, g].copy(), want, f"rowwise scales of group {g}")
        lo = hi
    _no_nan_codes(q)


def test_moe_bwd_rowwise_transposed_view_is_identical():
    """grad_out^T handed over as a transposed view of a row-major grad_out."""
    go = workloads.moe_grad_out_t()
    offs = workloads.moe_offsets()
    q1, s1 = jagged_rowwise(bf16_dev(go), i32_dev(offs))
    base = bf16_dev(np.ascontiguousarray(go.T))          # grad_out (16384, 4096) row-major
    q2, s2 = jagged_rowwise(base.t(), i32_dev(offs))
    assert np.array_equal(q1, q2)
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))


def test_moe_bwd_colwise_x():
    x = workloads.moe_x()
    offs = workloads.moe_offsets()
    q, s = jagged_colwise(bf16_dev(x), i32_dev(offs))
    cols = _sample(x.shape[1], 40, 2)
    oq, os_ = oracle.quantize_jagged_colwise(np.ascontiguousarray(x[:, cols]), offs, canary=CANARY)
    assert_same_bytes(q[:, cols], oq, "moe_bwd colwise q (sampled columns)")
    assert_same_bytes(s[:, cols], os_, "moe_bwd colwise scales (sampled columns)")
    mag = x & 0x7FFF
    lo = 0
    for g, hi in enumerate(offs.tolist()):
        amax = mag[lo:hi].max(axis=0) if hi > lo else np.zeros(x.shape[1], np.uint16)
        want = _fp32_scales_from_amax_bits(amax)
        assert_same_bytes(s[g].copy(), want, f"colwise scales of group {g}")
        lo = hi
    _no_nan_codes(q)


@pytest.mark.parametrize("mode", ["floor", "rceil"])
def test_mx3d_e8(mode):
    E, N, K = 8, 8192, 5120
    w = np.stack([workloads.mx3d_expert(e) for e in range(E)])
    q, s = mx_3d_colwise(bf16_dev(w), mode=mode)
    ks = _sample(K, 24, 3)
    for e in (0, 3, 7):
        oq, os_ = oracle.quantize_mx_3d_colwise(np.ascontiguousarray(w[e:e + 1][:, :, ks]), mode=mode)
        assert_same_bytes(q[e:e + 1][:, :, ks], oq, f"mx3d q expert {e} (sampled columns)")
        assert_same_bytes(s[e:e + 1][:, :, ks], os_, f"mx3d scales expert {e} (sampled columns)")
    _no_nan_codes(q)


@pytest.mark.timeout(600)
def test_mx3d_sweep_prefixes_up_to_e64():
    """E in {1, 2, 4, 16, 64} at (E, 8192, 5120) with zero and 2^20 blocks.
    The E=64 run is checked against the oracle on sampled experts/columns,
    and every smaller E must reproduce the first E experts of it."""
    N, K = 8192, 5120
    Emax = 64
    dev_w = torch.empty((Emax, N, K), dtype=torch.bfloat16, device="cuda")
    host = {}
    for e in range(Emax):
        bits = workloads.mx3d_sweep_expert(e)
        dev_w[e].copy_(bf16_dev(bits))
        if e in (0, 1, 15, 63):
            host[e] = bits
    q64, s64 = mx_3d_colwise(dev_w)
    ks = _sample(K, 16, 4)
    for e, bits in host.items():
        oq, os_ = oracle.quantize_mx_3d_colwise(np.ascontiguousarray(bits[None][:, :, ks]))
        assert_same_bytes(q64[e:e + 1][:, :, ks], oq, f"sweep q expert {e}")
        assert_same_bytes(s64[e:e + 1][:, :, ks], os_, f"sweep scales expert {e}")
    assert (s64 == 0).sum() > 0                      # all-zero blocks hit the minimum code
    _no_nan_codes(q64)
    for E in (1, 2, 4, 16):
        qE, sE = mx_3d_colwise(dev_w[:E])
        assert np.array_equal(qE, q64[:E]), E
        assert np.array_equal(sE, s64[:E]), E


def test_blockwise_act_1x128():
    a = workloads.blockwise_act()
    q, s = blockwise(bf16_dev(a), 1, 128)
    rows = _sample(a.shape[0], 40, 5)
    oq, os_ = oracle.quantize_blockwise(a[rows], 1, 128)
    assert_same_bytes(q[rows], oq, "blockwise 1x128 q (sampled rows)")
    assert_same_bytes(s[rows], os_, "blockwise 1x128 scales (sampled rows)")
    amax = (a & 0x7FFF).reshape(a.shape[0], -1, 128).max(axis=2)
    assert_same_bytes(s, _fp32_scales_from_amax_bits(amax), "blockwise 1x128 all scales")
    _no_nan_codes(q)


def test_blockwise_weight_128x128():
    w = workloads.blockwise_weight()
    q, s = blockwise(bf16_dev(w), 128, 128)
    for rb in (0, 13, 31):
        sl = slice(128 * rb, 128 * rb + 128)
        oq, os_ = oracle.quantize_blockwise(np.ascontiguousarray(w[sl]), 128, 128)
        assert_same_bytes(q[sl], oq, f"blockwise 128x128 q (block row {rb})")
        assert_same_bytes(s[rb:rb + 1], os_, f"blockwise 128x128 scales (block row {rb})")
    amax = (w & 0x7FFF).reshape(32, 128, 32, 128).max(axis=(1, 3))
    assert_same_bytes(s, _fp32_scales_from_amax_bits(amax), "blockwise 128x128 all scales")
    _no_nan_codes(q)
