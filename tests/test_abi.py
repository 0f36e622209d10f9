"""CPU-side checks of the C-ABI library: it loads, exports every entry point
that include/mxq.h declares, and rejects bad arguments on the host before any
launch (these calls never reach the GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxq_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from mxfp8_quantization_moe_amd import _capi
    from mxfp8_quantization_moe_amd import build

    if build.needs_build():
        build.build()
    return _capi.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("mxq_quantize_jagged_rowwise", "mxq_quantize_jagged_colwise",
                     "mxq_quantize_mx_3d_colwise", "mxq_quantize_blockwise",
                     "mxq_quantize_mx_rowwise", "mxq_abi_version", "mxq_status_string"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    from mxfp8_quantization_moe_amd import _capi

    assert set(declared_functions()) == set(_capi.SIGNATURES)


def test_version_and_status_strings(lib):
    from mxfp8_quantization_moe_amd import _capi

    assert lib.mxq_abi_version() == 1
    assert _capi.status_string(0) == "MXQ_OK"
    assert _capi.status_string(1) == "MXQ_ERR_INVALID_ARG"
    assert _capi.status_string(2) == "MXQ_ERR_UNSUPPORTED"
    assert _capi.status_string(3) == "MXQ_ERR_LAUNCH"
    assert _capi.status_string(99) == "MXQ_ERR_UNKNOWN"


# Fake, never-dereferenced device addresses: every call below must return
# from host validation before touching the GPU.
A = 1 << 20          # 16-byte aligned
MIS = A + 2          # misaligned


def test_jagged_rejects_bad_arguments(lib):
    rw = lib.mxq_quantize_jagged_rowwise
    cw = lib.mxq_quantize_jagged_colwise
    ok_args = dict(x=A, rows=4, cols=64, sx_r=64, sx_c=1, offs=A, G=2, q=A, sq_r=64, sq_c=1, s=A,
                   ss0=2, ss1=1)

    def call(fn, **kw):
        a = dict(ok_args, **kw)
        return fn(a["x"], a["rows"], a["cols"], a["sx_r"], a["sx_c"], a["offs"], a["G"], a["q"],
                  a["sq_r"], a["sq_c"], a["s"], a["ss0"], a["ss1"], None)

    assert call(rw, G=0) == 1
    assert call(rw, G=4097) == 1
    assert call(rw, rows=-1) == 1
    assert call(rw, offs=0) == 1
    assert call(rw, s=0) == 1
    assert call(rw, x=0) == 1
    assert call(rw, x=MIS) == 1
    assert call(rw, q=A + 8) == 1
    assert call(rw, s=A + 2) == 1
    assert call(rw, sx_r=68) == 1                 # row stride not a multiple of 16 bytes
    assert call(rw, sx_c=2, sx_r=128) == 2        # no unit stride: no kernel
    assert call(rw, sx_c=2, sx_r=1) == 1          # transposed view, misaligned column stride
    assert call(rw, rows=0) == 0                  # nothing to do, no launch
    # colwise: row-major in, column-major out needs cols % 8 == 0
    assert call(cw, sq_r=1, sq_c=16, cols=12, sx_r=16) == 1
    assert call(cw, sq_r=64, sq_c=1) == 2         # row-major out from row-major in: no kernel
    assert call(cw, cols=0) == 0


def test_mx_and_blockwise_reject_bad_arguments(lib):
    mx3 = lib.mxq_quantize_mx_3d_colwise
    assert mx3(A, 2, 48, 64, 48 * 64, 64, 1, A, 48 * 64, 1, 48, A, 64, 64, 1, 0, None) == 1  # N % 32
    assert mx3(A, 0, 64, 64, 64 * 64, 64, 1, A, 64 * 64, 1, 64, A, 128, 64, 1, 1, None) == 0  # rceil
    assert mx3(A, 2, 64, 64, 64 * 64, 64, 1, A, 64 * 64, 1, 64, A, 128, 64, 1, -1, None) == 1  # mode
    assert mx3(A, 2, 64, 64, 64 * 64, 64, 1, A, 64 * 64, 1, 64, A, 128, 64, 1, 7, None) == 1  # mode
    assert mx3(A, 2, 64, 64, 64 * 64, 1, 64, A, 64 * 64, 1, 64, A, 128, 64, 1, 0, None) == 2  # layout
    assert mx3(A, 2, 64, 12, 64 * 12, 12, 1, A, 64 * 16, 1, 16, A, 24, 12, 1, 0, None) == 1  # K % 8
    assert mx3(0, 2, 64, 64, 64 * 64, 64, 1, A, 64 * 64, 1, 64, A, 128, 64, 1, 0, None) == 1  # null
    assert mx3(A, 0, 64, 64, 64 * 64, 64, 1, A, 64 * 64, 1, 64, A, 128, 64, 1, 0, None) == 0  # E = 0
    mxr = lib.mxq_quantize_mx_rowwise
    assert mxr(A, 4, 48, 48, 1, A, 48, 1, A, 1, 1, 0, None) == 1                        # cols % 32
    assert mxr(A, 0, 64, 64, 1, A, 64, 1, A, 2, 1, 1, None) == 0                        # rceil
    assert mxr(A, 4, 64, 64, 1, A, 64, 1, A, 2, 1, 2, None) == 1                        # mode
    bw = lib.mxq_quantize_blockwise
    assert bw(A, 128, 256, 256, 1, 1, 64, A, 256, 1, A, 4, 1, None) == 2                # 1x64
    assert bw(A, 100, 256, 256, 1, 128, 128, A, 1, 112, A, 2, 1, None) == 1             # rows % 128
    assert bw(A, 128, 256, 512, 2, 1, 128, A, 256, 1, A, 2, 1, None) == 2               # x: no unit stride
    assert bw(A, 128, 256, 256, 1, 128, 128, A, 512, 2, A, 2, 1, None) == 2             # q: no unit stride
    assert bw(A, 120, 256, 256, 1, 1, 128, A, 1, 128, A, 2, 1, None) == 1               # 1x128 col-major, rows % 16
    assert bw(A, 256, 120, 1, 256, 128, 1, A, 120, 1, A, 120, 1, None) == 1             # its transposed view
    assert bw(A, 128, 256, 256, 1, 128, 128, A, 252, 1, A, 2, 1, None) == 1             # row-major q pitch % 8
    assert bw(A, 0, 256, 256, 1, 128, 128, A, 1, 16, A, 2, 1, None) == 0                # empty


def test_jagged_mx_rejects_bad_arguments(lib):
    rw = lib.mxq_quantize_jagged_mx_rowwise
    cw = lib.mxq_quantize_jagged_mx_colwise
    ok_args = dict(x=A, rows=4, cols=64, sx_r=64, sx_c=1, offs=A, G=2, q=A, sq_r=64, sq_c=1, s=A,
                   ss0=3, ss1=1, mode=0)

    def call(fn, **kw):
        a = dict(ok_args, **kw)
        return fn(a["x"], a["rows"], a["cols"], a["sx_r"], a["sx_c"], a["offs"], a["G"], a["q"],
                  a["sq_r"], a["sq_c"], a["s"], a["ss0"], a["ss1"], a["mode"], None)

    assert call(rw, G=0) == 1
    assert call(rw, G=4097) == 1
    assert call(rw, mode=2) == 1
    assert call(rw, offs=0) == 1
    assert call(rw, s=0) == 1
    assert call(rw, q=MIS) == 1
    assert call(rw, sx_r=60) == 1                  # row pitch not a multiple of 8
    assert call(rw, sx_r=1, sx_c=3) == 1           # transposed view, misaligned pitch
    assert call(rw, sx_r=1, sx_c=64, rows=6) == 1  # transposed view needs rows % 8 == 0
    assert call(rw, sq_r=1, sq_c=4) == 2           # column-major out: no kernel
    assert call(rw, cols=0) == 0 and call(rw, rows=0, mode=1) == 0
    assert call(cw, sq_r=1, sq_c=16, cols=12, sx_r=16) == 1   # cols % 8
    assert call(cw, sq_r=64, sq_c=1) == 2          # row-major out from row-major in: no kernel
    assert call(cw, rows=0, sq_r=1, sq_c=16) == 0


def test_relayout_rejects_bad_arguments(lib):
    fn = lib.mxq_relayout_mx_scales_grouped
    ok_args = dict(s=A, rows=32, ss_r=40, ss_b=1, offs=A, G=2, extent=1000, tiles=A, starts=A)

    def call(**kw):
        a = dict(ok_args, **kw)
        return fn(a["s"], a["rows"], a["ss_r"], a["ss_b"], a["offs"], a["G"], a["extent"],
                  a["tiles"], a["starts"], None)

    assert call(G=0) == 1
    assert call(G=4097) == 1
    assert call(offs=0) == 1
    assert call(rows=-1) == 1
    assert call(extent=-5) == 1
    assert call(ss_r=-40) == 1
    assert call(s=0) == 1
    assert call(tiles=0) == 1
    assert call(tiles=MIS) == 1                    # tiles must be 16-byte aligned
    assert call(starts=A + 2) == 1                 # tile_starts must be 4-byte aligned
    assert call(rows=1 << 31) == 1
    assert call(rows=(1 << 31) - 16, extent=(1 << 31) - 1) == 1   # tile numbers past int32
    assert call(rows=0, starts=0) == 0             # nothing to write: no launch
