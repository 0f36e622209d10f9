"""The C ABI from plain C: tests/c_abi_check.c includes only include/mxq.h and
the HIP runtime API, compiles with gcc as C11 with warnings as errors and
links against libmxq.so (and the oracle for its comparisons).  The GPU test
runs it."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
PKG = os.path.join(ROOT, "mxfp8_quantization_moe_amd")
ORACLE = os.path.join(ROOT, "oracle")


def _build(tmp_path):
    from mxfp8_quantization_moe_amd import build

    if build.needs_build():
        build.build()
    import oracle

    oracle.build()
    exe = str(tmp_path / "c_abi_check")
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "c_abi_check.c"), "-o", exe,
           "-L", PKG, "-lmxq", "-L", ORACLE, "-loracle", "-L", os.path.join(ROCM, "lib"),
           "-lamdhip64", f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{ORACLE}",
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


def test_c_program_compiles_and_links(tmp_path):
    assert os.path.exists(_build(tmp_path))


@pytest.mark.gpu
def test_c_program_matches_oracle(tmp_path):
    exe = _build(tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c abi check: ok" in r.stdout
