"""Helpers for the GPU tests: device buffers from the shared seeded inputs and
direct calls of the C-ABI entry points with caller-allocated, canary-filled
outputs.  Results come back as numpy arrays in logical index order, ready to
compare byte for byte with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import mxfp8_quantization_moe_amd as mxq
import workloads

CANARY = 0xA5
DEV = torch.device("cuda:0")


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    """Device bf16 tensor with the given bit patterns.  The last dim is padded
    in storage to a multiple of 8 elements (16 bytes), as the library requires
    16-byte aligned rows; the returned view has the logical shape."""
    bits = np.ascontiguousarray(bits)
    t = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    last = bits.shape[-1] if bits.ndim else 0
    if bits.ndim >= 2 and last % 8 != 0:
        ld = (last + 7) // 8 * 8
        padded = torch.zeros(bits.shape[:-1] + (ld,), dtype=torch.bfloat16, device=DEV)
        padded[..., :last].copy_(t)
        t = padded[..., :last]
    return t


def i32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(DEV)


def u8_canary(n: int) -> torch.Tensor:
    return torch.full((max(n, 1),), CANARY, dtype=torch.uint8, device=DEV)


def f32_canary(n: int) -> torch.Tensor:
    return torch.full((max(n, 1),), float("nan"), dtype=torch.float32, device=DEV)


def stream_handle(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(DEV)
    return s.cuda_stream


def _gather_u8(buf: torch.Tensor, shape, strides) -> np.ndarray:
    return buf.as_strided(shape, strides).cpu().numpy()


def _gather_f32(buf: torch.Tensor, shape, strides) -> np.ndarray:
    return buf.as_strided(shape, strides).cpu().numpy()


def round16(n: int) -> int:
    return (n + 15) // 16 * 16


def jagged_rowwise(x: torch.Tensor, offs: torch.Tensor, stream=None, expect=0):
    """Row-major q (row stride padded to 16 bytes), scales (rows, G)."""
    rows, cols = x.shape
    G = offs.numel()
    ldq = round16(max(cols, 1))
    q = u8_canary(rows * ldq)
    s = f32_canary(rows * G)
    code = mxq.mxq_quantize_jagged_rowwise(x.data_ptr(), rows, cols, x.stride(0), x.stride(1),
                                           offs.data_ptr(), G, q.data_ptr(), ldq, 1, s.data_ptr(),
                                           G, 1, stream_handle(stream))
    assert code == expect, code
    torch.cuda.synchronize()
    return _gather_u8(q, (rows, cols), (ldq, 1)), _gather_f32(s, (rows, G), (G, 1))


def jagged_colwise(x: torch.Tensor, offs: torch.Tensor, colmajor_out=True, stream=None, expect=0):
    """Column-major q (column stride padded), scales (G, cols)."""
    rows, cols = x.shape
    G = offs.numel()
    ldq = round16(max(rows, 1))
    q = u8_canary(cols * ldq)
    s = f32_canary(G * cols)
    code = mxq.mxq_quantize_jagged_colwise(x.data_ptr(), rows, cols, x.stride(0), x.stride(1),
                                           offs.data_ptr(), G, q.data_ptr(), 1, ldq, s.data_ptr(),
                                           cols, 1, stream_handle(stream))
    assert code == expect, code
    torch.cuda.synchronize()
    return _gather_u8(q, (rows, cols), (1, ldq)), _gather_f32(s, (G, cols), (cols, 1))


SCALE_MODES = {"floor": 0, "rceil": 1}


def mx_3d_colwise(w: torch.Tensor, stream=None, expect=0, mode="floor"):
    """Per-expert column-major q (E, N, K) strides (K*ldn, 1, ldn); scales
    (E, N/32, K) contiguous."""
    E, N, K = w.shape
    ldn = round16(N)
    q = u8_canary(E * K * ldn)
    s = u8_canary(E * (N // 32) * K)
    code = mxq.mxq_quantize_mx_3d_colwise(w.data_ptr(), E, N, K, w.stride(0), w.stride(1),
                                          w.stride(2), q.data_ptr(), K * ldn, 1, ldn, s.data_ptr(),
                                          (N // 32) * K, K, 1, SCALE_MODES[mode],
                                          stream_handle(stream))
    assert code == expect, code
    torch.cuda.synchronize()
    return (_gather_u8(q, (E, N, K), (K * ldn, 1, ldn)),
            _gather_u8(s, (E, N // 32, K), ((N // 32) * K, K, 1)))


def mx_rowwise(x: torch.Tensor, stream=None, expect=0, mode="floor"):
    rows, cols = x.shape
    ldq = round16(cols)
    q = u8_canary(rows * ldq)
    s = u8_canary(rows * (cols // 32))
    code = mxq.mxq_quantize_mx_rowwise(x.data_ptr(), rows, cols, x.stride(0), x.stride(1),
                                       q.data_ptr(), ldq, 1, s.data_ptr(), cols // 32, 1,
                                       SCALE_MODES[mode], stream_handle(stream))
    assert code == expect, code
    torch.cuda.synchronize()
    return _gather_u8(q, (rows, cols), (ldq, 1)), _gather_u8(s, (rows, cols // 32), (cols // 32, 1))


def blockwise(x: torch.Tensor, br: int, bc: int, stream=None, expect=0, qlayout=None):
    """q row-major (qlayout "row"; the default for 1 x 128) or column-major
    ("col"; the default otherwise), pitch padded to 16 bytes; scales
    (rows/br, cols/bc) row-major.  x may be any view with a unit stride."""
    rows, cols = x.shape
    nrb, ncb = rows // br, cols // bc
    s = f32_canary(nrb * ncb)
    if qlayout is None:
        qlayout = "row" if br == 1 else "col"
    if qlayout == "row":
        ldq = round16(cols)
        q = u8_canary(rows * ldq)
        qs = (ldq, 1)
    else:
        ldq = round16(rows)
        q = u8_canary(cols * ldq)
        qs = (1, ldq)
    code = mxq.mxq_quantize_blockwise(x.data_ptr(), rows, cols, x.stride(0), x.stride(1), br, bc,
                                      q.data_ptr(), qs[0], qs[1], s.data_ptr(), ncb, 1,
                                      stream_handle(stream))
    assert code == expect, code
    torch.cuda.synchronize()
    return _gather_u8(q, (rows, cols), qs), _gather_f32(s, (nrb, ncb), (ncb, 1))


def assert_same_bytes(got: np.ndarray, want: np.ndarray, what: str) -> None:
    """Byte-exact comparison with the first mismatches reported by index."""
    if got.dtype == np.float32:
        got = got.view(np.uint32)
        want = want.view(np.uint32)
    if np.array_equal(got, want):
        return
    bad = np.argwhere(got != want)
    head = ", ".join(f"{tuple(int(i) for i in b)}: got {got[tuple(b)]:#x} want {want[tuple(b)]:#x}"
                     for b in bad[:10])
    raise AssertionError(f"{what}: {len(bad)} mismatches; first: {head}")


def jagged_mx_rowwise(x: torch.Tensor, offs: torch.Tensor, mode="floor", stream=None, expect=0):
    """Row-major q (row stride padded to 16 bytes), scales (rows, capacity)."""
    rows, cols = x.shape
    G = offs.numel()
    nb = mxq.jagged_mx_scale_capacity(cols, G)
    ldq = round16(max(cols, 1))
    q = u8_canary(rows * ldq)
    s = u8_canary(rows * nb)
    code = mxq.mxq_quantize_jagged_mx_rowwise(x.data_ptr(), rows, cols, x.stride(0), x.stride(1),
                                              offs.data_ptr(), G, q.data_ptr(), ldq, 1,
                                              s.data_ptr(), nb, 1, SCALE_MODES[mode],
                                              stream_handle(stream))
    assert code == expect, code
    torch.cuda.synchronize()
    return _gather_u8(q, (rows, cols), (ldq, 1)), _gather_u8(s, (rows, nb), (nb, 1))


def jagged_mx_colwise(x: torch.Tensor, offs: torch.Tensor, mode="floor", stream=None, expect=0):
    """Column-major q (column stride padded), scales (capacity, cols)."""
    rows, cols = x.shape
    G = offs.numel()
    nb = mxq.jagged_mx_scale_capacity(rows, G)
    ldq = round16(max(rows, 1))
    q = u8_canary(cols * ldq)
    s = u8_canary(nb * cols)
    code = mxq.mxq_quantize_jagged_mx_colwise(x.data_ptr(), rows, cols, x.stride(0), x.stride(1),
                                              offs.data_ptr(), G, q.data_ptr(), 1, ldq,
                                              s.data_ptr(), cols, 1, SCALE_MODES[mode],
                                              stream_handle(stream))
    assert code == expect, code
    torch.cuda.synchronize()
    return _gather_u8(q, (rows, cols), (1, ldq)), _gather_u8(s, (nb, cols), (cols, 1))


def adversarial(shape, seed):
    """N(0,1) bf16 with 1/16 of the entries replaced by signed zeros,
    subnormals, the largest finite values, exact powers of two and values
    that land on e4m3 rounding ties."""
    g = np.random.default_rng(seed)
    bits = workloads.normal_bf16(shape, seed)
    flat = bits.reshape(-1)
    pick = g.choice(flat.size, size=max(1, flat.size // 16), replace=False)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F,
                         0x3F80, 0xBF80, 0x43E0, 0x3C00], dtype=np.uint16)
    flat[pick] = specials[g.integers(specials.size, size=pick.size)]
    return bits


def random_offsets(extent, G, seed, multiple=1, empties=1, short_tail=0):
    """Sorted random group ends on multiples of ``multiple``, with ``empties``
    forced empty groups and the last ``short_tail`` elements in no group."""
    g = np.random.default_rng(seed)
    cuts = np.sort(g.integers(0, (extent - short_tail) // multiple + 1, size=G - 1)) * multiple
    offs = np.concatenate([cuts, [extent - short_tail]]).astype(np.int64)
    for _ in range(empties):
        j = int(g.integers(1, G)) if G > 1 else 0
        if j > 0:
            offs[j] = offs[j - 1]
    offs = np.maximum.accumulate(offs)
    return offs.astype(np.int32)


def relayout(scales_dev, offs, extent, stream=None):
    """Direct C-ABI call of the scale re-layout with canary-filled outputs;
    returns (tiles up to capacity, tile_starts) as numpy."""
    rows = scales_dev.shape[0]
    G = len(offs)
    cap = mxq.mx_tile_capacity(rows, extent, G)
    tiles = torch.full((max(cap, 16),), CANARY, dtype=torch.uint8, device=DEV)
    starts = torch.full((G + 1,), -7, dtype=torch.int32, device=DEV)
    d_offs = i32_dev(offs)
    st = stream if stream is not None else torch.cuda.current_stream()
    code = mxq.mxq_relayout_mx_scales_grouped(
        scales_dev.data_ptr(), rows, scales_dev.stride(0), scales_dev.stride(1), d_offs.data_ptr(),
        G, extent, tiles.data_ptr(), starts.data_ptr(), st.cuda_stream)
    assert code == 0, mxq._capi.status_string(code)
    st.synchronize()
    return tiles.cpu().numpy()[:cap], starts.cpu().numpy()


def colwise_workspace(rows: int, cols: int, G: int) -> torch.Tensor:
    """A zero-filled workspace for the colwise call with a workspace."""
    n = mxq.mxq_jagged_colwise_workspace_bytes(rows, cols, G)
    assert n >= 0
    return torch.zeros(max(n, 4) // 4, dtype=torch.int32, device=DEV)


def jagged_colwise_ws(x: torch.Tensor, offs: torch.Tensor, ws: torch.Tensor, spin=None, stream=None,
                      expect=0, ws_bytes=None):
    """The colwise call with a workspace (``spin``: the test-only entry with
    that wait bound); column-major q (column stride padded), scales (G, cols)."""
    rows, cols = x.shape
    G = offs.numel()
    ldq = round16(max(rows, 1))
    q = u8_canary(cols * ldq)
    s = f32_canary(G * cols)
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    args = (x.data_ptr(), rows, cols, x.stride(0), x.stride(1), offs.data_ptr(), G, q.data_ptr(), 1,
            ldq, s.data_ptr(), cols, 1, ws.data_ptr(), nbytes)
    if spin is None:
        code = mxq.mxq_quantize_jagged_colwise_ws(*args, stream_handle(stream))
    else:
        code = mxq.mxq_debug_jagged_colwise_ws_spin(*args, spin, stream_handle(stream))
    assert code == expect, code
    torch.cuda.synchronize()
    return _gather_u8(q, (rows, cols), (1, ldq)), _gather_f32(s, (G, cols), (cols, 1))
