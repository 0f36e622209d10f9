"""ctypes declarations of the C ABI in include/mxq.h.

Argument marshalling only: every function here forwards plain integers
(device pointers, extents, strides, a stream handle) to ``libmxq.so`` and
returns its status code.  The library must have been built
(``python -m mxfp8_quantization_moe_amd.build`` or ``__graft_entry__.build()``);
there is no fallback of any kind when it is missing.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmxq.so")

MXQ_OK = 0
MXQ_ERR_INVALID_ARG = 1
MXQ_ERR_UNSUPPORTED = 2
MXQ_ERR_LAUNCH = 3
MXQ_ERR_WORKSPACE = 4
MXQ_SCALE_FLOOR = 0
MXQ_SCALE_RCEIL = 1
MXQ_MAX_GROUPS = 4096
MXQ_NOALLOC_SCRATCH_BYTES = 4 << 20

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_vp = ctypes.c_void_p
_st = ctypes.c_int

# name -> argument types (restype is mxq_status == int unless listed below)
SIGNATURES = {
    "mxq_abi_version": [],
    "mxq_status_string": [ctypes.c_int],
    "mxq_quantize_jagged_rowwise": [_vp, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _i64, _i64, _vp,
                                    _i64, _i64, _vp],
    "mxq_quantize_jagged_colwise": [_vp, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _i64, _i64, _vp,
                                    _i64, _i64, _vp],
    "mxq_quantize_mx_3d_colwise": [_vp, _i64, _i64, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _i64,
                                   _vp, _i64, _i64, _i64, _i32, _vp],
    "mxq_quantize_mx_rowwise": [_vp, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64,
                                _i32, _vp],
    "mxq_quantize_jagged_mx_rowwise": [_vp, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _i64, _i64,
                                       _vp, _i64, _i64, _i32, _vp],
    "mxq_quantize_jagged_mx_colwise": [_vp, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _i64, _i64,
                                       _vp, _i64, _i64, _i32, _vp],
    "mxq_relayout_mx_scales_grouped": [_vp, _i64, _i64, _i64, _vp, _i32, _i64, _vp, _vp, _vp],
    "mxq_quantize_blockwise": [_vp, _i64, _i64, _i64, _i64, _i32, _i32, _vp, _i64, _i64, _vp,
                               _i64, _i64, _vp],
    "mxq_quantize_jagged_colwise_ws": [_vp, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _i64, _i64,
                                       _vp, _i64, _i64, _vp, _i64, _vp],
    "mxq_jagged_colwise_workspace_bytes": [_i64, _i64, _i32],
    "mxq_quantize_jagged_colwise_noalloc": [_vp, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _i64,
                                            _i64, _vp, _i64, _i64, _vp],
    "mxq_debug_jagged_colwise_ws_spin": [_vp, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _i64, _i64,
                                         _vp, _i64, _i64, _vp, _i64, _i32, _vp],
    "mxq_debug_cast_e4m3": [_vp, _i64, _vp, _vp],
    "mxq_debug_cast4_e4m3": [_vp, _i64, _vp, _i32, _vp],
}
RESTYPES = {"mxq_status_string": ctypes.c_char_p, "mxq_jagged_colwise_workspace_bytes": _i64}

_lib = None


class LibraryMissing(RuntimeError):
    pass


def load() -> ctypes.CDLL:
    """Load libmxq.so (once).  Raises LibraryMissing if it was never built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(
            f"{LIB_PATH} is not built; run `python -m mxfp8_quantization_moe_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, args in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = RESTYPES.get(name, _st)
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().mxq_status_string(code).decode()


def _fwd(name):
    def call(*args):
        return getattr(load(), name)(*args)

    call.__name__ = name
    call.__doc__ = f"Direct call of the C entry point ``{name}`` (see include/mxq.h)."
    return call


mxq_abi_version = _fwd("mxq_abi_version")
mxq_quantize_jagged_rowwise = _fwd("mxq_quantize_jagged_rowwise")
mxq_quantize_jagged_colwise = _fwd("mxq_quantize_jagged_colwise")
mxq_quantize_mx_3d_colwise = _fwd("mxq_quantize_mx_3d_colwise")
mxq_quantize_mx_rowwise = _fwd("mxq_quantize_mx_rowwise")
mxq_quantize_jagged_mx_rowwise = _fwd("mxq_quantize_jagged_mx_rowwise")
mxq_quantize_jagged_mx_colwise = _fwd("mxq_quantize_jagged_mx_colwise")
mxq_relayout_mx_scales_grouped = _fwd("mxq_relayout_mx_scales_grouped")
mxq_quantize_blockwise = _fwd("mxq_quantize_blockwise")
mxq_quantize_jagged_colwise_ws = _fwd("mxq_quantize_jagged_colwise_ws")
mxq_jagged_colwise_workspace_bytes = _fwd("mxq_jagged_colwise_workspace_bytes")
mxq_debug_jagged_colwise_ws_spin = _fwd("mxq_debug_jagged_colwise_ws_spin")
mxq_quantize_jagged_colwise_noalloc = _fwd("mxq_quantize_jagged_colwise_noalloc")
mxq_debug_cast_e4m3 = _fwd("mxq_debug_cast_e4m3")
mxq_debug_cast4_e4m3 = _fwd("mxq_debug_cast4_e4m3")
