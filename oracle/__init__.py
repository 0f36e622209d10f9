"""Plain CPU oracle (ctypes wrapper around ``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the HIP library and
its Python binding never do, and share no code with it.

Every function takes bf16 inputs as ``numpy.uint16`` bit patterns (any
strides) and returns freshly allocated numpy outputs in *logical* index order:
``q[i, j]`` is the e4m3 byte of element ``(i, j)`` whatever memory layout the
GPU writes.  The C code follows the definitions cited in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
             "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile ``oracle.c`` with gcc into ``liboracle.so`` (always rebuilds)."""
    cmd = ["gcc", *GCC_FLAGS, "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


_lib = None

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_vp = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_e4m3_encode_array.argtypes = [_vp, _i64, _vp]
    lib.oracle_e4m3_encode_array.restype = None
    lib.oracle_fp32_scale.argtypes = [ctypes.c_float]
    lib.oracle_fp32_scale.restype = ctypes.c_float
    lib.oracle_e8m0_floor.argtypes = [ctypes.c_float]
    lib.oracle_e8m0_floor.restype = ctypes.c_uint8
    lib.oracle_e8m0_rceil.argtypes = [ctypes.c_float]
    lib.oracle_e8m0_rceil.restype = ctypes.c_uint8
    jag = [_vp, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _i64, _i64, _vp, _i64, _i64]
    lib.oracle_quantize_jagged_rowwise.argtypes = jag
    lib.oracle_quantize_jagged_colwise.argtypes = jag
    lib.oracle_quantize_mx_3d_colwise.argtypes = [_vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                                  _vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64,
                                                  ctypes.c_int]
    lib.oracle_quantize_mx_rowwise.argtypes = [_vp, _i64, _i64, _i64, _i64, _vp, _i64, _i64,
                                               _vp, _i64, _i64, ctypes.c_int]
    jmx = [_vp, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _i64, _i64, _vp, _i64, _i64, ctypes.c_int]
    lib.oracle_quantize_jagged_mx_rowwise.argtypes = jmx
    lib.oracle_quantize_jagged_mx_colwise.argtypes = jmx
    lib.oracle_quantize_blockwise.argtypes = [_vp, _i64, _i64, _i64, _i64, _i32, _i32, _vp,
                                              _i64, _i64, _vp, _i64, _i64]
    lib.oracle_relayout_mx_scales_grouped.argtypes = [_vp, _i64, _i64, _i64, _vp, _i32, _vp, _vp]
    for name in ("oracle_relayout_mx_scales_grouped", "oracle_quantize_jagged_rowwise", "oracle_quantize_jagged_colwise",
                 "oracle_quantize_mx_3d_colwise", "oracle_quantize_mx_rowwise",
                 "oracle_quantize_blockwise", "oracle_quantize_jagged_mx_rowwise",
                 "oracle_quantize_jagged_mx_colwise"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _estrides(a: np.ndarray):
    return tuple(s // a.itemsize for s in a.strides)


def _check_bf16(x: np.ndarray, ndim: int) -> None:
    if x.dtype != np.uint16 or x.ndim != ndim:
        raise TypeError(f"expected a {ndim}-D uint16 (bf16 bit pattern) array, got {x.dtype} {x.shape}")


def _call(status: int, what: str) -> None:
    if status != 0:
        raise ValueError(f"oracle rejected the arguments of {what}")


# ------------------------------------------------------------------ numerics

def e4m3_encode(y) -> np.ndarray:
    """Saturating RNE encode of float32 values into E4M3FN bytes."""
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float32))
    out = np.empty(y.shape, dtype=np.uint8)
    _load().oracle_e4m3_encode_array(_ptr(y), y.size, _ptr(out))
    return out


def e4m3_decode(codes) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    lib = _load()
    flat = [lib.oracle_e4m3_decode(int(c)) for c in codes.ravel()]
    return np.array(flat, dtype=np.float64).reshape(codes.shape)


def fp32_scale(amax) -> np.ndarray:
    lib = _load()
    a = np.asarray(amax, dtype=np.float32)
    flat = [lib.oracle_fp32_scale(float(v)) for v in a.ravel()]
    return np.array(flat, dtype=np.float32).reshape(a.shape)


def e8m0_floor(amax) -> np.ndarray:
    lib = _load()
    a = np.asarray(amax, dtype=np.float32)
    flat = [lib.oracle_e8m0_floor(float(v)) for v in a.ravel()]
    return np.array(flat, dtype=np.uint8).reshape(a.shape)


def e8m0_rceil(amax) -> np.ndarray:
    lib = _load()
    a = np.asarray(amax, dtype=np.float32)
    flat = [lib.oracle_e8m0_rceil(float(v)) for v in a.ravel()]
    return np.array(flat, dtype=np.uint8).reshape(a.shape)


SCALE_MODES = {"floor": 0, "rceil": 1}


# ---------------------------------------------------------- quantization ops

def quantize_jagged_rowwise(x: np.ndarray, offs, canary: int = 0):
    """x: (rows, cols) bf16 bits, groups along dim 1.  Returns (q, scales)
    with q (rows, cols) uint8 and scales (rows, G) float32.  Bytes in no group
    (at or past offs[-1]) keep ``canary``."""
    _check_bf16(x, 2)
    offs = np.ascontiguousarray(np.asarray(offs, dtype=np.int32))
    rows, cols = x.shape
    G = offs.size
    q = np.full((rows, cols), canary, dtype=np.uint8)
    s = np.zeros((rows, G), dtype=np.float32)
    sx = _estrides(x)
    _call(_load().oracle_quantize_jagged_rowwise(_ptr(x), rows, cols, sx[0], sx[1], _ptr(offs), G,
                                                 _ptr(q), cols, 1, _ptr(s), G, 1),
          "jagged_rowwise")
    return q, s


def quantize_jagged_colwise(x: np.ndarray, offs, canary: int = 0):
    """x: (rows, cols) bf16 bits, groups along dim 0.  Returns (q, scales)
    with q (rows, cols) uint8 and scales (G, cols) float32."""
    _check_bf16(x, 2)
    offs = np.ascontiguousarray(np.asarray(offs, dtype=np.int32))
    rows, cols = x.shape
    G = offs.size
    q = np.full((rows, cols), canary, dtype=np.uint8)
    s = np.zeros((G, cols), dtype=np.float32)
    sx = _estrides(x)
    _call(_load().oracle_quantize_jagged_colwise(_ptr(x), rows, cols, sx[0], sx[1], _ptr(offs), G,
                                                 _ptr(q), cols, 1, _ptr(s), cols, 1),
          "jagged_colwise")
    return q, s


def quantize_mx_3d_colwise(w: np.ndarray, mode: str = "floor"):
    """w: (E, N, K) bf16 bits.  Returns q (E, N, K) uint8 and e8m0 scales
    (E, N/32, K) uint8, both in logical index order.  mode: floor | rceil."""
    _check_bf16(w, 3)
    E, N, K = w.shape
    q = np.zeros((E, N, K), dtype=np.uint8)
    s = np.zeros((E, N // 32, K), dtype=np.uint8)
    sw = _estrides(w)
    _call(_load().oracle_quantize_mx_3d_colwise(_ptr(w), E, N, K, sw[0], sw[1], sw[2], _ptr(q),
                                                N * K, K, 1, _ptr(s), (N // 32) * K, K, 1,
                                                SCALE_MODES[mode]),
          "mx_3d_colwise")
    return q, s


def quantize_mx_rowwise(x: np.ndarray, mode: str = "floor"):
    """x: (rows, cols) bf16 bits, 1x32 blocks along dim 1.  Returns q (rows,
    cols) uint8 and e8m0 scales (rows, cols/32) uint8."""
    _check_bf16(x, 2)
    rows, cols = x.shape
    q = np.zeros((rows, cols), dtype=np.uint8)
    s = np.zeros((rows, cols // 32), dtype=np.uint8)
    sx = _estrides(x)
    _call(_load().oracle_quantize_mx_rowwise(_ptr(x), rows, cols, sx[0], sx[1], _ptr(q), cols, 1,
                                             _ptr(s), cols // 32, 1, SCALE_MODES[mode]),
          "mx_rowwise")
    return q, s


def jagged_mx_scale_capacity(extent: int, G: int) -> int:
    """Upper bound of sum_g ceil(n_g / 32) over any G groups covering at most
    ``extent`` elements: ceil(extent / 32) + G - 1."""
    return (extent + 31) // 32 + G - 1


def quantize_jagged_mx_rowwise(x: np.ndarray, offs, mode: str = "floor", canary: int = 0):
    """x: (rows, cols) bf16 bits, groups along dim 1, 1x32 blocks restarting
    at each group start.  Returns q (rows, cols) and e8m0 scales (rows,
    capacity) uint8; bytes and scale entries the op does not write keep
    ``canary``."""
    _check_bf16(x, 2)
    offs = np.ascontiguousarray(np.asarray(offs, dtype=np.int32))
    rows, cols = x.shape
    G = offs.size
    nb = jagged_mx_scale_capacity(cols, G)
    q = np.full((rows, cols), canary, dtype=np.uint8)
    s = np.full((rows, nb), canary, dtype=np.uint8)
    sx = _estrides(x)
    _call(_load().oracle_quantize_jagged_mx_rowwise(_ptr(x), rows, cols, sx[0], sx[1], _ptr(offs), G,
                                                    _ptr(q), cols, 1, _ptr(s), nb, 1,
                                                    SCALE_MODES[mode]),
          "jagged_mx_rowwise")
    return q, s


def quantize_jagged_mx_colwise(x: np.ndarray, offs, mode: str = "floor", canary: int = 0):
    """x: (rows, cols) bf16 bits, groups along dim 0, 32x1 blocks restarting
    at each group start.  Returns q (rows, cols) and e8m0 scales (capacity,
    cols) uint8; unwritten entries keep ``canary``."""
    _check_bf16(x, 2)
    offs = np.ascontiguousarray(np.asarray(offs, dtype=np.int32))
    rows, cols = x.shape
    G = offs.size
    nb = jagged_mx_scale_capacity(rows, G)
    q = np.full((rows, cols), canary, dtype=np.uint8)
    s = np.full((nb, cols), canary, dtype=np.uint8)
    sx = _estrides(x)
    _call(_load().oracle_quantize_jagged_mx_colwise(_ptr(x), rows, cols, sx[0], sx[1], _ptr(offs), G,
                                                    _ptr(q), cols, 1, _ptr(s), cols, 1,
                                                    SCALE_MODES[mode]),
          "jagged_mx_colwise")
    return q, s


def mx_tile_capacity(rows: int, extent: int, G: int) -> int:
    """Upper bound, in bytes, of the re-laid-out scales of ``rows`` rows and
    G groups covering at most ``extent`` tokens: 256 bytes per tile,
    ceil(rows/16) row blocks, at most ceil(extent/512) + G - 1 K tiles."""
    return 256 * ((rows + 15) // 16) * ((extent + 511) // 512 + G - 1) if G > 0 else 0


def relayout_mx_scales_grouped(scales: np.ndarray, offs, extent: int, canary: int = 0):
    """scales: (rows, blocks) uint8 e8m0 array (any strides) whose block b of
    row r is the jagged MX scale of that row and block, offs: the token
    groups of the jagged MX quantization that wrote them (covering at most
    ``extent`` tokens).  For the colwise operand pass the transposed (cols,
    blocks) view.  Returns the tile bytes (capacity bytes; bytes past the last
    tile keep ``canary``) and tile_starts (G + 1 int32)."""
    if scales.dtype != np.uint8 or scales.ndim != 2:
        raise TypeError("expected a 2-D uint8 array of e8m0 scales")
    offs = np.ascontiguousarray(np.asarray(offs, dtype=np.int32))
    rows = scales.shape[0]
    G = offs.size
    out = np.full(mx_tile_capacity(rows, extent, G), canary, dtype=np.uint8)
    starts = np.zeros(G + 1, dtype=np.int32)
    ss = scales.strides
    _call(_load().oracle_relayout_mx_scales_grouped(_ptr(scales), rows, ss[0], ss[1], _ptr(offs), G,
                                                    _ptr(out), _ptr(starts)),
          "relayout_mx_scales_grouped")
    return out, starts


def quantize_blockwise(x: np.ndarray, block_r: int, block_c: int):
    """x: (rows, cols) bf16 bits, block_r x block_c blocks.  Returns q (rows,
    cols) uint8 and scales (rows/block_r, cols/block_c) float32."""
    _check_bf16(x, 2)
    rows, cols = x.shape
    q = np.zeros((rows, cols), dtype=np.uint8)
    nrb, ncb = rows // block_r, cols // block_c
    s = np.zeros((nrb, ncb), dtype=np.float32)
    sx = _estrides(x)
    _call(_load().oracle_quantize_blockwise(_ptr(x), rows, cols, sx[0], sx[1], block_r, block_c,
                                            _ptr(q), cols, 1, _ptr(s), ncb, 1),
          "blockwise")
    return q, s
