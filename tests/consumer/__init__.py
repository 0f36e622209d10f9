"""Test-only HIP consumer of the scaled-MFMA scale tiles (built by
``build()``, loaded by the GPU tests)."""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "scaled_mfma_consumer.hip")
LIB = os.path.join(HERE, "libscaled_mfma_consumer.so")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def build(verbose: bool = False) -> str:
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", LIB + ".tmp", SRC]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def needs_build() -> bool:
    return not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC)


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built (run build())")
        lib = ctypes.CDLL(LIB)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.consumer_grouped_gemm.argtypes = [vp, i64, i32, vp, i64, i32, vp, vp, vp, vp, vp, i32, vp,
                                              i32, i32, i32, i32]
        lib.consumer_grouped_gemm.restype = ctypes.c_int
        _lib = lib
    return _lib
