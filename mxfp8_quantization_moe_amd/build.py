"""Build ``libmxq.so`` (the HIP kernels behind the C ABI in include/mxq.h).

The library is compiled in-tree with hipcc for gfx950 only.  Flags:
IEEE fp32 division and denormals are kept (no fast-math), no FMA contraction,
and packed-fp32 instruction selection is switched off.
"""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmxq.so")
SOURCES = [os.path.join(CSRC, "api.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("mxq_device.hpp", "wave_ops.hpp", "jagged_kernels.hpp",
                                            "jagged_mx_kernels.hpp", "block_kernels.hpp", "group_tables.hpp",
                                            "colwise_tile_kernels.hpp",
                                            "relayout_kernels.hpp")] + [os.path.join(ROOT, "include", "mxq.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fno-gpu-rdc",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False, extra=()) -> str:
    """Compile the library (always rebuilds); returns the path of the .so."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


def needs_build() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
