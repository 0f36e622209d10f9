"""The colwise entry point that allocates nothing
(mxq_quantize_jagged_colwise_noalloc, scratch in a device array inside the
library) against the entry point it varies (mxq_quantize_jagged_colwise_ws
with a fresh workspace), byte for byte, on two calls in a row, the second
on a smaller input; both also against the oracle.  Extents whose scratch
would exceed the array are refused before any launch."""
import numpy as np
import pytest
import torch

import mxfp8_quantization_moe_amd as mxq
import oracle
import workloads
from gpu_helpers import (CANARY, DEV, adversarial, assert_same_bytes, bf16_dev, colwise_workspace,
                         i32_dev, jagged_colwise_ws, round16, stream_handle)

pytestmark = pytest.mark.gpu


def noalloc(x, offs, expect=0):
    rows, cols = x.shape
    G = offs.numel()
    ldq = round16(max(rows, 1))
    q = torch.full((cols * ldq,), CANARY, dtype=torch.uint8, device=DEV)
    s = torch.full((G * cols,), float("nan"), dtype=torch.float32, device=DEV)
    code = mxq.mxq_quantize_jagged_colwise_noalloc(
        x.data_ptr(), rows, cols, x.stride(0), x.stride(1), offs.data_ptr(), G, q.data_ptr(), 1, ldq,
        s.data_ptr(), cols, 1, stream_handle())
    assert code == expect, mxq._capi.status_string(code)
    torch.cuda.synchronize()
    return (q.as_strided((rows, cols), (1, ldq)).cpu().numpy(),
            s.view(G, cols).cpu().numpy())


def test_two_calls_in_a_row_match_the_workspace_entry_point():
    big = workloads.moe_x()                                   # (16384, 4096), the MoE groups
    cases = [(big, workloads.moe_offsets()),
             (adversarial((7000, 520), 4000), np.array([3, 3, 5000, 6990], np.int32))]
    for k, (bits, offs) in enumerate(cases):
        x, d_offs = bf16_dev(bits), i32_dev(offs)
        q, s = noalloc(x, d_offs)
        ws = colwise_workspace(*bits.shape, len(offs))
        wq, wsc = jagged_colwise_ws(x, d_offs, ws)
        assert_same_bytes(q, wq, f"call {k} q against the workspace entry point")
        assert_same_bytes(s, wsc, f"call {k} scales against the workspace entry point")
        cols = np.r_[0:64, bits.shape[1] - 64:bits.shape[1]]  # first and last strips vs the oracle
        oq, os_ = oracle.quantize_jagged_colwise(np.ascontiguousarray(bits[:, cols]), offs, canary=CANARY)
        assert_same_bytes(q[:, cols], oq, f"call {k} q against the oracle")
        assert_same_bytes(s[:, cols], os_, f"call {k} scales against the oracle")


def test_refuses_extents_beyond_the_array():
    x = bf16_dev(adversarial((64, 64), 4001))
    d_offs = i32_dev([64])
    rows, cols = 65536, 65536
    need = mxq.mxq_jagged_colwise_workspace_bytes(rows, cols, 1)
    assert need > mxq.MXQ_NOALLOC_SCRATCH_BYTES
    q = torch.empty(16, dtype=torch.uint8, device=DEV)
    s = torch.empty(4, dtype=torch.float32, device=DEV)
    code = mxq.mxq_quantize_jagged_colwise_noalloc(x.data_ptr(), rows, cols, cols, 1, d_offs.data_ptr(),
                                                   1, q.data_ptr(), 1, rows, s.data_ptr(), cols, 1,
                                                   stream_handle())
    assert code == mxq.MXQ_ERR_WORKSPACE


def test_many_groups_need_no_scratch():
    """More than 256 groups run the kernel without chunks: no scratch is
    needed, any extent is accepted, and the result is the oracle's."""
    bits = adversarial((9000, 64), 4002)
    offs = np.sort(np.random.default_rng(4002).integers(0, 9001, 300)).astype(np.int32)
    offs[-1] = 9000
    assert mxq.mxq_jagged_colwise_workspace_bytes(9000, 64, 300) == 0
    q, s = noalloc(bf16_dev(bits), i32_dev(offs))
    oq, os_ = oracle.quantize_jagged_colwise(bits, offs, canary=CANARY)
    assert_same_bytes(q, oq, "many groups q")
    assert_same_bytes(s, os_, "many groups scales")
