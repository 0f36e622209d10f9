"""Host-side behaviour of the Python binding: it refuses tensors the kernels
cannot take before any call reaches the library, and without a built
library it fails loudly (there is no CPU fallback of any kind)."""
import os

import pytest
import torch

import mxfp8_quantization_moe_amd as mxq
from mxfp8_quantization_moe_amd import _capi


def test_cpu_and_wrong_dtype_tensors_are_refused():
    x_cpu = torch.zeros((4, 64), dtype=torch.bfloat16)
    offs = torch.tensor([64], dtype=torch.int32)
    for fn in (mxq.quantize_jagged_rowwise, mxq.quantize_jagged_colwise,
               mxq.quantize_jagged_mx_rowwise, mxq.quantize_jagged_mx_colwise):
        with pytest.raises(TypeError):
            fn(x_cpu, offs)
    with pytest.raises(TypeError):
        mxq.quantize_mx_rowwise(x_cpu)
    with pytest.raises(TypeError):
        mxq.quantize_blockwise(x_cpu, 1, 128)
    with pytest.raises(TypeError):
        mxq.quantize_mx_3d_colwise(torch.zeros((1, 32, 8), dtype=torch.float32))


def test_missing_library_raises(tmp_path, monkeypatch):
    monkeypatch.setattr(_capi, "LIB_PATH", str(tmp_path / "libmxq.so"))
    monkeypatch.setattr(_capi, "_lib", None)
    assert not os.path.exists(_capi.LIB_PATH)
    with pytest.raises(_capi.LibraryMissing):
        _capi.load()
    with pytest.raises(_capi.LibraryMissing):
        mxq.mxq_abi_version()
