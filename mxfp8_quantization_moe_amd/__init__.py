"""mxq: dynamic float8 (OCP E4M3FN) quantization of MoE grouped-GEMM operands
on AMD Instinct MI355X (gfx950).

Thin tensor-level binding over the C ABI in ``include/mxq.h``: each function
validates nothing beyond what is needed to marshal arguments, allocates the
outputs with torch on the input's device, and forwards device pointers,
extents, strides and the current HIP stream to ``libmxq.so``.  Every step of
the computation runs in the library's HIP kernels; there is no CPU path.

Outputs ``q`` are ``torch.float8_e4m3fn`` tensors laid out as the grouped GEMM
consumes them (row-major or column-major, see each function); fp32 scales are
quantize multipliers ``448 / max(amax, 1e-12)``; e8m0 scales are
``torch.uint8`` biased exponents.
"""
from __future__ import annotations

from . import _capi
from ._capi import (MXQ_ERR_INVALID_ARG, MXQ_ERR_LAUNCH, MXQ_ERR_UNSUPPORTED, MXQ_ERR_WORKSPACE,
                    MXQ_MAX_GROUPS, mxq_debug_jagged_colwise_ws_spin,
                    mxq_jagged_colwise_workspace_bytes, mxq_quantize_jagged_colwise_ws,
                    mxq_quantize_jagged_colwise_noalloc, MXQ_NOALLOC_SCRATCH_BYTES,
                    MXQ_OK, MXQ_SCALE_FLOOR, MXQ_SCALE_RCEIL, LibraryMissing,
                    mxq_abi_version, mxq_debug_cast4_e4m3, mxq_debug_cast_e4m3,
                    mxq_quantize_blockwise,
                    mxq_quantize_jagged_colwise, mxq_quantize_jagged_mx_colwise,
                    mxq_quantize_jagged_mx_rowwise, mxq_quantize_jagged_rowwise,
                    mxq_quantize_mx_3d_colwise, mxq_quantize_mx_rowwise,
                    mxq_relayout_mx_scales_grouped)

__all__ = [
    "quantize_jagged_rowwise", "quantize_jagged_colwise", "quantize_mx_3d_colwise",
    "quantize_mx_rowwise", "quantize_jagged_mx_rowwise", "quantize_jagged_mx_colwise",
    "jagged_mx_scale_capacity", "relayout_mx_scales_grouped", "mx_tile_capacity",
    "quantize_blockwise", "debug_cast_e4m3", "MXQError",
    "mxq_quantize_jagged_rowwise", "mxq_quantize_jagged_colwise", "mxq_quantize_mx_3d_colwise",
    "mxq_quantize_mx_rowwise", "mxq_quantize_jagged_mx_rowwise", "mxq_quantize_jagged_mx_colwise",
    "mxq_relayout_mx_scales_grouped", "mxq_quantize_blockwise", "mxq_debug_cast_e4m3",
    "mxq_debug_cast4_e4m3", "debug_cast4_e4m3", "jagged_colwise_workspace",
    "mxq_quantize_jagged_colwise_ws", "mxq_jagged_colwise_workspace_bytes",
    "mxq_debug_jagged_colwise_ws_spin", "mxq_quantize_jagged_colwise_noalloc",
    "mxq_abi_version", "LibraryMissing",
]


class MXQError(ValueError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {_capi.status_string(code)}")
        self.code = code


def _torch():
    import torch
    return torch


def _stream(t, stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(code: int, what: str) -> None:
    if code != MXQ_OK:
        raise MXQError(code, what)


def _require_bf16_cuda(x, ndim: int, name: str):
    torch = _torch()
    if x.dtype != torch.bfloat16 or x.dim() != ndim or not x.is_cuda:
        raise TypeError(f"{name} must be a {ndim}-D bfloat16 CUDA tensor, got {x.dtype} "
                        f"{tuple(x.shape)} on {x.device}")


def _require_offs(offs, x):
    """Group ends: a contiguous 1-D int32 tensor on x's device (read only by
    the kernels, never on the host)."""
    torch = _torch()
    if (offs.dtype != torch.int32 or offs.dim() != 1 or not offs.is_contiguous()
            or offs.device != x.device):
        raise TypeError(f"offs must be a contiguous 1-D int32 tensor on {x.device}, got "
                        f"{offs.dtype} {tuple(offs.shape)} on {offs.device}")


def _round_up(n: int, m: int) -> int:
    return (n + m - 1) // m * m


def _empty_rowmajor_u8(torch, rows: int, cols: int, device):
    """(rows, cols) float8 tensor whose row stride is a multiple of 16 bytes."""
    ld = _round_up(max(cols, 1), 16)
    buf = torch.empty(rows * ld, dtype=torch.float8_e4m3fn, device=device)
    return buf.as_strided((rows, cols), (ld, 1))


def _empty_colmajor_u8(torch, rows: int, cols: int, device):
    """(rows, cols) float8 tensor stored column-major with a 16-byte-multiple
    column stride."""
    ld = _round_up(max(rows, 1), 16)
    buf = torch.empty(cols * ld, dtype=torch.float8_e4m3fn, device=device)
    return buf.as_strided((rows, cols), (1, ld))


def quantize_jagged_rowwise(x, offs, *, stream=None):
    """Per-(row, group) scaling with groups along dim 1 of ``x`` (rows, cols).

    ``offs``: int32 CUDA tensor of cumulative group ends (never read on the
    host).  Returns ``(q, scales)``: q (rows, cols) row-major e4m3, scales
    (rows, G) fp32.  ``x`` may be row-major or the transpose of a row-major
    tensor (e.g. ``grad_out.t()``)."""
    torch = _torch()
    _require_bf16_cuda(x, 2, "x")
    _require_offs(offs, x)
    rows, cols = x.shape
    G = offs.numel()
    q = _empty_rowmajor_u8(torch, rows, cols, x.device)
    s = torch.empty((rows, G), dtype=torch.float32, device=x.device)
    code = mxq_quantize_jagged_rowwise(
        x.data_ptr(), rows, cols, x.stride(0), x.stride(1), offs.data_ptr(), G, q.data_ptr(),
        q.stride(0), q.stride(1), s.data_ptr(), s.stride(0), s.stride(1), _stream(x, stream))
    _check(code, "mxq_quantize_jagged_rowwise")
    return q, s


def jagged_colwise_workspace(rows: int, cols: int, num_groups: int, device=None):
    """A zero-filled workspace for ``quantize_jagged_colwise(...,
    workspace=ws)`` on (rows, cols) with num_groups groups.  Every call
    leaves it zero-filled, so it can be kept and reused by calls that do not
    overlap in time."""
    torch = _torch()
    n = mxq_jagged_colwise_workspace_bytes(rows, cols, num_groups)
    if n < 0:
        raise MXQError(MXQ_ERR_INVALID_ARG, "mxq_jagged_colwise_workspace_bytes")
    return torch.zeros(max(n, 4) // 4, dtype=torch.int32, device=device or "cuda")


def quantize_jagged_colwise(x, offs, *, workspace=None, stream=None):
    """Per-(group, column) scaling with groups along dim 0 of ``x`` (rows,
    cols).  Returns ``(q, scales)``: q (rows, cols) column-major e4m3, scales
    (G, cols) fp32.  With a ``workspace`` (``jagged_colwise_workspace``),
    groups longer than one workgroup's rows are split across workgroups and
    every element is read once."""
    torch = _torch()
    _require_bf16_cuda(x, 2, "x")
    _require_offs(offs, x)
    rows, cols = x.shape
    G = offs.numel()
    q = _empty_colmajor_u8(torch, rows, cols, x.device)
    s = torch.empty((G, cols), dtype=torch.float32, device=x.device)
    args = (x.data_ptr(), rows, cols, x.stride(0), x.stride(1), offs.data_ptr(), G, q.data_ptr(),
            q.stride(0), q.stride(1), s.data_ptr(), s.stride(0), s.stride(1))
    if workspace is None:
        _check(mxq_quantize_jagged_colwise(*args, _stream(x, stream)), "mxq_quantize_jagged_colwise")
    else:
        if not workspace.is_cuda or workspace.device != x.device or not workspace.is_contiguous():
            raise TypeError("workspace must be a contiguous CUDA tensor on x's device")
        nbytes = workspace.numel() * workspace.element_size()
        _check(mxq_quantize_jagged_colwise_ws(*args, workspace.data_ptr(), nbytes, _stream(x, stream)),
               "mxq_quantize_jagged_colwise_ws")
    return q, s


def quantize_mx_3d_colwise(w, *, scale_mode: int = MXQ_SCALE_FLOOR, stream=None):
    """MXFP8 along N of expert weights ``w`` (E, N, K).  Returns ``(q,
    scales)``: q (E, N, K) with per-expert column-major strides (N*K, 1, N)
    (the column stride N rounded up to 16 bytes), scales (E, N/32, K) e8m0
    uint8."""
    torch = _torch()
    _require_bf16_cuda(w, 3, "w")
    E, N, K = w.shape
    ldk = _round_up(max(N, 1), 16)
    buf = torch.empty(E * K * ldk, dtype=torch.float8_e4m3fn, device=w.device)
    q = buf.as_strided((E, N, K), (K * ldk, 1, ldk))
    s = torch.empty((E, N // 32, K), dtype=torch.uint8, device=w.device)
    code = mxq_quantize_mx_3d_colwise(
        w.data_ptr(), E, N, K, w.stride(0), w.stride(1), w.stride(2), q.data_ptr(), q.stride(0),
        q.stride(1), q.stride(2), s.data_ptr(), s.stride(0), s.stride(1), s.stride(2), scale_mode,
        _stream(w, stream))
    _check(code, "mxq_quantize_mx_3d_colwise")
    return q, s


def quantize_mx_rowwise(x, *, scale_mode: int = MXQ_SCALE_FLOOR, stream=None):
    """MXFP8 in 1x32 blocks along dim 1.  Returns ``(q, scales)``: q (rows,
    cols) row-major e4m3, scales (rows, cols/32) e8m0 uint8."""
    torch = _torch()
    _require_bf16_cuda(x, 2, "x")
    rows, cols = x.shape
    q = _empty_rowmajor_u8(torch, rows, cols, x.device)
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    code = mxq_quantize_mx_rowwise(
        x.data_ptr(), rows, cols, x.stride(0), x.stride(1), q.data_ptr(), q.stride(0), q.stride(1),
        s.data_ptr(), s.stride(0), s.stride(1), scale_mode, _stream(x, stream))
    _check(code, "mxq_quantize_mx_rowwise")
    return q, s


def jagged_mx_scale_capacity(extent: int, num_groups: int) -> int:
    """Scale entries a jagged MX call may write along the grouped dim:
    ceil(extent/32) + num_groups - 1, the most that any offsets need."""
    return (extent + 31) // 32 + num_groups - 1


def quantize_jagged_mx_rowwise(x, offs, *, scale_mode: int = MXQ_SCALE_FLOOR, stream=None):
    """MXFP8 with 1x32 blocks restarting at each group start, groups along
    dim 1.  Returns ``(q, scales)``: q (rows, cols) row-major e4m3, scales
    (rows, capacity) e8m0 uint8 where the first sum_g ceil(n_g/32) columns
    are written."""
    torch = _torch()
    _require_bf16_cuda(x, 2, "x")
    _require_offs(offs, x)
    rows, cols = x.shape
    G = offs.numel()
    q = _empty_rowmajor_u8(torch, rows, cols, x.device)
    s = torch.empty((rows, jagged_mx_scale_capacity(cols, G)), dtype=torch.uint8, device=x.device)
    code = mxq_quantize_jagged_mx_rowwise(
        x.data_ptr(), rows, cols, x.stride(0), x.stride(1), offs.data_ptr(), G, q.data_ptr(),
        q.stride(0), q.stride(1), s.data_ptr(), s.stride(0), s.stride(1), scale_mode,
        _stream(x, stream))
    _check(code, "mxq_quantize_jagged_mx_rowwise")
    return q, s


def quantize_jagged_mx_colwise(x, offs, *, scale_mode: int = MXQ_SCALE_FLOOR, stream=None):
    """MXFP8 with 32x1 blocks restarting at each group start, groups along
    dim 0.  Returns ``(q, scales)``: q (rows, cols) column-major e4m3, scales
    (capacity, cols) e8m0 uint8 where the first sum_g ceil(n_g/32) rows are
    written."""
    torch = _torch()
    _require_bf16_cuda(x, 2, "x")
    _require_offs(offs, x)
    rows, cols = x.shape
    G = offs.numel()
    q = _empty_colmajor_u8(torch, rows, cols, x.device)
    s = torch.empty((jagged_mx_scale_capacity(rows, G), cols), dtype=torch.uint8, device=x.device)
    code = mxq_quantize_jagged_mx_colwise(
        x.data_ptr(), rows, cols, x.stride(0), x.stride(1), offs.data_ptr(), G, q.data_ptr(),
        q.stride(0), q.stride(1), s.data_ptr(), s.stride(0), s.stride(1), scale_mode,
        _stream(x, stream))
    _check(code, "mxq_quantize_jagged_mx_colwise")
    return q, s


def mx_tile_capacity(rows: int, extent: int, num_groups: int) -> int:
    """Bytes of scaled-MFMA scale tiles that a re-layout of ``rows`` rows and
    ``num_groups`` groups over ``extent`` tokens may write:
    256 * ceil(rows/16) * (ceil(extent/512) + num_groups - 1)."""
    return 256 * ((rows + 15) // 16) * ((extent + 511) // 512 + num_groups - 1)


def relayout_mx_scales_grouped(scales, offs, extent: int, *, stream=None):
    """Per-group re-layout of jagged MX scales into scaled-MFMA scale tiles.
    ``scales``: (rows, blocks) uint8 e8m0 tensor, any strides (for the colwise
    operand pass the (cols, blocks) transposed view of its scales), ``offs``
    and ``extent``: the groups and the token extent of the jagged MX call.
    Returns ``(tiles, tile_starts)``: tiles a uint8 tensor of
    mx_tile_capacity bytes (tile_starts[G] * 256 of them written),
    tile_starts (G + 1,) int32."""
    torch = _torch()
    if scales.dtype != torch.uint8 or scales.dim() != 2 or not scales.is_cuda:
        raise TypeError(f"scales must be a 2-D uint8 CUDA tensor, got {scales.dtype} "
                        f"{tuple(scales.shape)} on {scales.device}")
    _require_offs(offs, scales)
    rows = scales.shape[0]
    G = offs.numel()
    tiles = torch.empty(max(mx_tile_capacity(rows, extent, G), 16), dtype=torch.uint8,
                        device=scales.device)
    starts = torch.empty(G + 1, dtype=torch.int32, device=scales.device)
    code = mxq_relayout_mx_scales_grouped(
        scales.data_ptr(), rows, scales.stride(0), scales.stride(1), offs.data_ptr(), G, extent,
        tiles.data_ptr(), starts.data_ptr(), _stream(scales, stream))
    _check(code, "mxq_relayout_mx_scales_grouped")
    return tiles, starts


def quantize_blockwise(x, block_r: int, block_c: int, *, stream=None):
    """Blockwise fp8 with one fp32 multiplier per block.  (1, 128): q row-major;
    (128, 128) and (128, 1): q column-major.  Returns ``(q, scales)`` with
    scales (rows/block_r, cols/block_c) fp32."""
    torch = _torch()
    _require_bf16_cuda(x, 2, "x")
    rows, cols = x.shape
    if block_r == 1:
        q = _empty_rowmajor_u8(torch, rows, cols, x.device)
    else:
        q = _empty_colmajor_u8(torch, rows, cols, x.device)
    s = torch.empty((rows // block_r, cols // block_c), dtype=torch.float32, device=x.device)
    code = mxq_quantize_blockwise(
        x.data_ptr(), rows, cols, x.stride(0), x.stride(1), block_r, block_c, q.data_ptr(),
        q.stride(0), q.stride(1), s.data_ptr(), s.stride(0), s.stride(1), _stream(x, stream))
    _check(code, "mxq_quantize_blockwise")
    return q, s


def debug_cast_e4m3(y, *, stream=None):
    """The library's device cast (saturate, RNE to E4M3FN) on an fp32 CUDA
    tensor; returns uint8 codes."""
    torch = _torch()
    if y.dtype != torch.float32 or not y.is_cuda or not y.is_contiguous():
        raise TypeError("y must be a contiguous float32 CUDA tensor")
    out = torch.empty(y.shape, dtype=torch.uint8, device=y.device)
    _check(mxq_debug_cast_e4m3(y.data_ptr(), y.numel(), out.data_ptr(), _stream(y, stream)),
           "mxq_debug_cast_e4m3")
    return out


def debug_cast4_e4m3(y, unclamped: bool, *, stream=None):
    """Test-only: the packed conversion of the quantization kernels on an fp32
    CUDA tensor, four values at a time; ``unclamped`` selects the form of
    the fp32-multiplier paths (defined for |y| < 464 only), else the clamped
    form of the e8m0 paths.  Returns uint8 codes."""
    torch = _torch()
    if y.dtype != torch.float32 or not y.is_cuda or not y.is_contiguous():
        raise TypeError("y must be a contiguous float32 CUDA tensor")
    out = torch.empty(y.shape, dtype=torch.uint8, device=y.device)
    _check(mxq_debug_cast4_e4m3(y.data_ptr(), y.numel(), out.data_ptr(), 1 if unclamped else 0,
                                _stream(y, stream)), "mxq_debug_cast4_e4m3")
    return out
