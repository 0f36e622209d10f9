"""Parity on tensors of more than 2^31 elements, where every address offset
needs 64-bit arithmetic: the jagged rowwise / colwise, jagged MX and
blockwise entry points, checked against the oracle on sampled rows or
columns (each sample a complete reduction unit) plus the scale of every
group.  The MX 3D kernel's 2^31+ case is the E=64 sweep of the full-size
configuration tests."""
import numpy as np
import pytest
import torch

import mxfp8_quantization_moe_amd as mxq
import oracle
import workloads
from gpu_helpers import assert_same_bytes, i32_dev

pytestmark = pytest.mark.gpu

BIG = (1 << 31) + (1 << 20)      # elements, just past 2^31


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _u8(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def _rows(q: torch.Tensor, r: torch.Tensor) -> np.ndarray:
    """Bytes of rows r of an e4m3 / uint8 tensor (any strides)."""
    return _u8(q.view(torch.uint8).index_select(0, r))


def _cols(q: torch.Tensor, c: torch.Tensor) -> np.ndarray:
    return _u8(q.view(torch.uint8).index_select(1, c))


def _sample(n, k, seed):
    g = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], g.choice(n, size=k, replace=False)]))


def test_jagged_rowwise_past_2_31():
    rows, cols = 65600, 32768                    # 2.15e9 elements
    assert rows * cols > BIG - (1 << 21)
    x = workloads.device_normal_bf16((rows, cols), 11)
    offs = np.array([5000, 5000, 19000, 32768], dtype=np.int32)
    q, s = mxq.quantize_jagged_rowwise(x, i32_dev(offs))
    torch.cuda.synchronize()
    r = torch.from_numpy(_sample(rows, 6, 1)).cuda()
    xb = _bits(x.index_select(0, r))
    oq, os_ = oracle.quantize_jagged_rowwise(xb, offs)
    assert_same_bytes(_rows(q, r), oq, "rowwise q (sampled rows)")
    assert_same_bytes(s.index_select(0, r).cpu().numpy(), os_, "rowwise scales (sampled rows)")
    del x, q, s


def test_jagged_colwise_past_2_31():
    rows, cols = 262400, 8192                    # 2.15e9 elements, column-major q
    x = workloads.device_normal_bf16((rows, cols), 12)
    offs = np.array([100000, 100016, 200000, 262400], dtype=np.int32)
    q, s = mxq.quantize_jagged_colwise(x, i32_dev(offs))
    torch.cuda.synchronize()
    c = torch.from_numpy(_sample(cols, 5, 2)).cuda()
    xb = _bits(x.index_select(1, c))
    oq, os_ = oracle.quantize_jagged_colwise(xb, offs)
    assert_same_bytes(_cols(q, c), oq, "colwise q (sampled columns)")
    assert_same_bytes(s.index_select(1, c).cpu().numpy(), os_, "colwise scales (sampled columns)")
    del x, q, s


def test_jagged_mx_past_2_31():
    rows, cols = 262400, 8192
    x = workloads.device_normal_bf16((rows, cols), 13)
    offs = np.array([100000, 100016, 200000, 262400], dtype=np.int32)
    q, s = mxq.quantize_jagged_mx_colwise(x, i32_dev(offs), scale_mode=mxq.MXQ_SCALE_RCEIL)
    torch.cuda.synchronize()
    c = torch.from_numpy(_sample(cols, 4, 3)).cuda()
    xb = _bits(x.index_select(1, c))
    oq, os_ = oracle.quantize_jagged_mx_colwise(xb, offs, mode="rceil")
    nb = sum((int(n) + 31) // 32 for n in np.diff(np.concatenate([[0], offs])))
    assert_same_bytes(_cols(q, c), oq, "jagged mx q (sampled columns)")
    assert_same_bytes(_cols(s, c)[:nb], os_[:nb], "jagged mx scales (sampled columns)")
    del x, q, s


def test_blockwise_past_2_31():
    rows, cols = 65600, 32768
    x = workloads.device_normal_bf16((rows, cols), 14)
    q, s = mxq.quantize_blockwise(x, 1, 128)
    torch.cuda.synchronize()
    r = torch.from_numpy(_sample(rows, 6, 4)).cuda()
    xb = _bits(x.index_select(0, r))
    oq, os_ = oracle.quantize_blockwise(xb, 1, 128)
    assert_same_bytes(_rows(q, r), oq, "blockwise q (sampled rows)")
    assert_same_bytes(s.index_select(0, r).cpu().numpy(), os_, "blockwise scales (sampled rows)")
    del x, q, s
