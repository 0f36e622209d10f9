"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer.

``oracle_sanitize_driver.c`` and ``oracle/oracle.c`` are compiled together
with ``-fsanitize=address,undefined`` (errors abort); every oracle function
then runs on edge cases (empty groups, groups past the extent's end, one
group, many groups, strided and transposed inputs, zero blocks, every
bf16 amax) with each buffer allocated at exactly the size the call may
touch.  The sanitized build must run clean and give byte for byte the
output of the normal build, whose results the other oracle tests pin."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CANARY = 0xA5

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("san") / "oracle_sanitize_driver")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fno-fast-math", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"),
           "-o", exe, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr or "").lower():
        pytest.skip("no AddressSanitizer runtime: " + r.stderr[-300:])
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


def run(driver, tmp_path, op, blobs, *args):
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        for b in blobs:
            f.write(np.ascontiguousarray(b).tobytes())
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([driver, op, str(src), str(dst), *[str(int(a)) for a in args]],
                       capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"{op}: rc {r.returncode}\n{r.stderr[-4000:]}"
    return dst.read_bytes()


def strided(bits, layout):
    """A view of ``bits`` with the same logical values and its backing
    buffer: row-major, a transposed view, or every other column of a wider
    buffer."""
    if layout == "row":
        base = np.ascontiguousarray(bits)
        return base, base
    if layout == "t":
        base = np.ascontiguousarray(bits.T)
        return base.T, base
    base = np.zeros((bits.shape[0], 2 * bits.shape[1] + 1), dtype=np.uint16)
    base[:, 0:2 * bits.shape[1]:2] = bits
    return base[:, 0:2 * bits.shape[1]:2], base


def estrides(v):
    return [s // v.itemsize for s in v.strides]


def adversarial(shape, seed):
    g = np.random.default_rng(seed)
    bits = workloads.normal_bf16(shape, seed)
    flat = bits.reshape(-1)
    pick = g.choice(flat.size, size=max(1, flat.size // 8), replace=False)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x7F7F, 0xFF7F, 0x3F80, 0x43E0],
                        dtype=np.uint16)
    flat[pick] = specials[g.integers(specials.size, size=pick.size)]
    return bits


OFFS = {  # extent -> group ends: empty groups, a short tail, one group, many groups
    "mixed": lambda n: np.array([0, n // 3, n // 3, n - 5], dtype=np.int32),
    "one": lambda n: np.array([n], dtype=np.int32),
    "many": lambda n: np.sort(np.random.default_rng(n).integers(0, n + 1, size=70)).astype(np.int32),
}


@pytest.mark.parametrize("layout", ["row", "t", "gap"])
@pytest.mark.parametrize("kind", list(OFFS))
def test_jagged_fp32(driver, tmp_path, layout, kind):
    x = adversarial((37, 83), 1)
    v, base = strided(x, layout)
    for op, ext in (("jagged_rowwise", 83), ("jagged_colwise", 37)):
        offs = OFFS[kind](ext)
        G = offs.size
        got = run(driver, tmp_path, op, [base, offs], 37, 83, *estrides(v), G, base.size)
        fn = oracle.quantize_jagged_rowwise if op == "jagged_rowwise" else oracle.quantize_jagged_colwise
        q, s = fn(v, offs, canary=CANARY)
        assert got == q.tobytes() + s.tobytes(), (op, layout, kind)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("kind", list(OFFS))
def test_jagged_mx(driver, tmp_path, mode, kind):
    x = adversarial((41, 150), 2)
    name = ("floor", "rceil")[mode]
    for layout in ("row", "t"):
        v, base = strided(x, layout)
        for op, ext in (("jagged_mx_rowwise", 150), ("jagged_mx_colwise", 41)):
            offs = OFFS[kind](ext)
            got = run(driver, tmp_path, op, [base, offs], 41, 150, *estrides(v), offs.size, base.size, mode)
            fn = (oracle.quantize_jagged_mx_rowwise if op == "jagged_mx_rowwise"
                  else oracle.quantize_jagged_mx_colwise)
            q, s = fn(v, offs, mode=name, canary=CANARY)
            assert got == q.tobytes() + s.tobytes(), (op, layout, kind, mode)


@pytest.mark.parametrize("mode", [0, 1])
def test_mx_3d_and_rowwise(driver, tmp_path, mode):
    name = ("floor", "rceil")[mode]
    w = adversarial((3, 64, 40), 3)
    w[1, :32, 5] = 0                                           # a zero block
    got = run(driver, tmp_path, "mx3d", [w], 3, 64, 40, 64 * 40, 40, 1, w.size, mode)
    q, s = oracle.quantize_mx_3d_colwise(w, mode=name)
    assert got == q.tobytes() + s.tobytes()
    wt = np.ascontiguousarray(w.transpose(0, 2, 1))           # (E, K, N) storage, N innermost
    v = wt.transpose(0, 2, 1)
    got = run(driver, tmp_path, "mx3d", [wt], 3, 64, 40, 64 * 40, 1, 64, wt.size, mode)
    q, s = oracle.quantize_mx_3d_colwise(v, mode=name)
    assert got == q.tobytes() + s.tobytes()
    x = adversarial((19, 96), 4)
    for layout in ("row", "t", "gap"):
        v, base = strided(x, layout)
        got = run(driver, tmp_path, "mx_rowwise", [base], 19, 96, *estrides(v), base.size, mode)
        q, s = oracle.quantize_mx_rowwise(v, mode=name)
        assert got == q.tobytes() + s.tobytes(), layout


@pytest.mark.parametrize("br,bc", [(1, 128), (128, 128), (128, 1)])
def test_blockwise(driver, tmp_path, br, bc):
    x = adversarial((256, 384), 5)
    x[:br, :bc] = 0
    for layout in ("row", "t", "gap"):
        v, base = strided(x, layout)
        got = run(driver, tmp_path, "blockwise", [base], 256, 384, *estrides(v), br, bc, base.size)
        q, s = oracle.quantize_blockwise(v, br, bc)
        assert got == q.tobytes() + s.tobytes(), layout


@pytest.mark.parametrize("kind", list(OFFS))
def test_relayout(driver, tmp_path, kind):
    extent = 3000
    offs = OFFS[kind](extent)
    G = offs.size
    cap = oracle.jagged_mx_scale_capacity(extent, G)
    sc = workloads.e8m0_bytes((37, cap), 6)
    t_base = np.ascontiguousarray(sc.T)
    gap = np.zeros((37, 2 * cap), dtype=np.uint8)
    gap[:, ::2] = sc
    for base, view in ((sc, sc), (t_base, t_base.T), (gap, gap[:, ::2])):
        got = run(driver, tmp_path, "relayout", [base, offs], 37, view.strides[0], view.strides[1], G,
                  extent, base.size)
        t, st = oracle.relayout_mx_scales_grouped(view, offs, extent, canary=CANARY)
        assert got == t.tobytes() + st.tobytes(), kind


def test_encode_and_scales(driver, tmp_path):
    g = np.random.default_rng(7)
    y = np.concatenate([
        (np.arange(0x7F800000, step=4099, dtype=np.int64)).astype(np.uint32).view(np.float32),
        (g.standard_normal(50_000) * 300).astype(np.float32),
        np.array([448.0, 464.0, 480.0, 1e30, -0.0, 2.0 ** -10, 3 * 2.0 ** -10], np.float32)])
    y = np.concatenate([y, -y])
    got = run(driver, tmp_path, "encode", [y], y.size)
    assert got == oracle.e4m3_encode(y).tobytes()
    got = np.frombuffer(run(driver, tmp_path, "scales", [], 0), dtype=np.uint8).reshape(-1, 6)
    b = np.arange(0x8000, dtype=np.uint32)
    b = b[((b >> 7) & 0xFF) != 0xFF]
    amax = (b << 16).view(np.float32)
    assert got.shape[0] == amax.size
    assert np.array_equal(got[:, :4].copy().view(np.float32).ravel().view(np.uint32),
                          oracle.fp32_scale(amax).view(np.uint32))
    assert np.array_equal(got[:, 4], oracle.e8m0_floor(amax))
    assert np.array_equal(got[:, 5], oracle.e8m0_rceil(amax))
