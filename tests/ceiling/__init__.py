"""Streaming probes for the practical HBM ceiling of the quantization
kernels' traffic mixes (2 bytes read + 1 byte written per element; 1:1 for the
scale re-layout), built by
``build()`` and timed by ``bench.py`` next to the kernels.  Bench and test
infrastructure: not part of the library."""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "stream_ceiling.hip")
LIB = os.path.join(HERE, "libstream_ceiling.so")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")

MODES = {"read2_write1": 0, "read_only": 1, "write_only": 2, "read2_write1_device_scope": 3,
         "read1_write1": 4}


def build(verbose: bool = False) -> str:
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", LIB + ".tmp", SRC]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built (run build())")
        lib = ctypes.CDLL(LIB)
        lib.ceiling_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                       ctypes.c_void_p]
        lib.ceiling_stream.restype = ctypes.c_int
        _lib = lib
    return _lib


def bytes_moved(n: int, mode: str) -> int:
    return {"read2_write1": 3 * n, "read_only": 2 * n, "write_only": n,
            "read2_write1_device_scope": 3 * n, "read1_write1": 4 * n}[mode]
