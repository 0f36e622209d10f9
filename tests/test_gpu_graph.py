"""The entry points under HIP graph capture: every call of one MoE backward
step plus the MX, blockwise and scale re-layout calls is captured into one
graph, which is replayed several times with unrelated eager work and
synchronisations in between; every replay must reproduce the eager outputs
byte for byte.
Nothing in the library allocates or records a memset, so capture needs no
special entry point."""
import numpy as np
import pytest
import torch

import mxfp8_quantization_moe_amd as mxq
import workloads
from gpu_helpers import bf16_dev, i32_dev

pytestmark = pytest.mark.gpu


def _calls(x_row, x_col, offs, w3, act):
    """(function, args without stream, output tensors) for each call."""
    R1, C1 = x_row.shape
    R2, C2 = x_col.shape
    G = offs.numel()
    E, N, K = w3.shape
    M, Ka = act.shape
    dev = x_row.device
    outs = {
        "q1": torch.full((R1 * C1,), 0xA5, dtype=torch.uint8, device=dev),
        "s1": torch.full((R1 * G,), float("nan"), dtype=torch.float32, device=dev),
        "q2": torch.full((R2 * C2,), 0xA5, dtype=torch.uint8, device=dev),
        "s2": torch.full((G * C2,), float("nan"), dtype=torch.float32, device=dev),
        "q3": torch.full((E * N * K,), 0xA5, dtype=torch.uint8, device=dev),
        "s3": torch.full((E * (N // 32) * K,), 0xA5, dtype=torch.uint8, device=dev),
        "q4": torch.full((M * Ka,), 0xA5, dtype=torch.uint8, device=dev),
        "s4": torch.full((M * (Ka // 128),), float("nan"), dtype=torch.float32, device=dev),
    }
    nb = mxq.jagged_mx_scale_capacity(R2, G)
    outs["q5"] = torch.full((R2 * C2,), 0xA5, dtype=torch.uint8, device=dev)
    outs["s5"] = torch.full((nb * C2,), 0xA5, dtype=torch.uint8, device=dev)
    outs["t6"] = torch.full((mxq.mx_tile_capacity(C2, R2, G),), 0xA5, dtype=torch.uint8, device=dev)
    outs["st6"] = torch.full((G + 1,), -1, dtype=torch.int32, device=dev)
    o = outs
    calls = [
        (mxq.mxq_quantize_jagged_rowwise,
         (x_row.data_ptr(), R1, C1, C1, 1, offs.data_ptr(), G, o["q1"].data_ptr(), C1, 1,
          o["s1"].data_ptr(), G, 1)),
        (mxq.mxq_quantize_jagged_colwise,
         (x_col.data_ptr(), R2, C2, C2, 1, offs.data_ptr(), G, o["q2"].data_ptr(), 1, R2,
          o["s2"].data_ptr(), C2, 1)),
        (mxq.mxq_quantize_mx_3d_colwise,
         (w3.data_ptr(), E, N, K, N * K, K, 1, o["q3"].data_ptr(), N * K, 1, N, o["s3"].data_ptr(),
          (N // 32) * K, K, 1, 0)),
        (mxq.mxq_quantize_blockwise,
         (act.data_ptr(), M, Ka, Ka, 1, 1, 128, o["q4"].data_ptr(), Ka, 1, o["s4"].data_ptr(),
          Ka // 128, 1)),
        (mxq.mxq_quantize_jagged_mx_colwise,
         (x_col.data_ptr(), R2, C2, C2, 1, offs.data_ptr(), G, o["q5"].data_ptr(), 1, R2,
          o["s5"].data_ptr(), C2, 1, 1)),
        # the scales just written, re-laid out for the scaled-MFMA consumer
        # (the columns of x are the rows of its scale matrix)
        (mxq.mxq_relayout_mx_scales_grouped,
         (o["s5"].data_ptr(), C2, 1, C2, offs.data_ptr(), G, R2, o["t6"].data_ptr(),
          o["st6"].data_ptr())),
    ]
    return calls, outs


def _run(calls, stream):
    for fn, args in calls:
        assert fn(*args, stream.cuda_stream) == 0


def _snapshot(outs):
    return {k: v.cpu().numpy().view(np.uint8).copy() for k, v in outs.items()}


def test_captured_step_replays_match_eager():
    a, _ = workloads.small_rowwise()          # (256, 1024), groups along its 1024 columns
    b, offs_b = workloads.small_colwise()     # (1024, 256), groups along its 1024 rows
    x_row, x_col = bf16_dev(a), bf16_dev(b)
    offs = i32_dev(offs_b)                    # one set of 1024-token groups for both
    w3 = bf16_dev(np.stack([workloads.mx3d_sweep_expert(e, N=256, K=512) for e in range(2)]))
    act = bf16_dev(workloads.normal_bf16((256, 512), 8))

    calls, outs = _calls(x_row, x_col, offs, w3, act)
    # one poison byte everywhere, before the eager run and before every
    # replay: entries a call does not write (scale capacity past the last
    # jagged MX block) hold it in both, and a replay that writes nothing fails
    for t in outs.values():
        t.view(torch.uint8).fill_(0x5A)
    stream = torch.cuda.current_stream()
    _run(calls, stream)
    torch.cuda.synchronize()
    eager = _snapshot(outs)

    for t in outs.values():
        t.view(torch.uint8).fill_(0x5A)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        _run(calls, torch.cuda.current_stream())
    torch.cuda.synchronize()

    scratch = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        for t in outs.values():
            t.view(torch.uint8).fill_(0x5A)
        scratch.mul_(1.0001).add_(0.5)     # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(outs)
        for k in eager:
            assert np.array_equal(got[k], eager[k]), f"replay {rep}: {k} differs from eager"
