"""The parallel oracle runner used by the full-size GPU parity tests: its
pieces, put back together, are the one-process oracle's output byte for
byte (every split is at reduction-unit boundaries)."""
import numpy as np
import pytest

import oracle
import oracle_pool
import workloads


def adversarial_bits(shape, seed):
    """N(0,1) bf16 bits with signed zeros, subnormals and the extremes mixed in."""
    g = np.random.default_rng(seed)
    bits = workloads.normal_bf16(shape, seed)
    flat = bits.reshape(-1)
    pick = g.choice(flat.size, size=flat.size // 8, replace=False)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x7F7F, 0xFF7F, 0x3F80, 0x43E0],
                        dtype=np.uint16)
    flat[pick] = specials[g.integers(specials.size, size=pick.size)]
    return bits


def offsets_with_tail(extent, G, tail):
    """G sorted group ends with one empty group and ``tail`` elements past the last."""
    g = np.random.default_rng(extent + G)
    cuts = np.sort(g.integers(0, extent - tail + 1, size=G - 1))
    offs = np.concatenate([cuts, [extent - tail]])
    offs[2] = offs[1]
    return np.maximum.accumulate(offs).astype(np.int32)


def same(a, b):
    a, b = np.asarray(a), np.asarray(b)
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), b.view(np.uint32)
    return a.shape == b.shape and np.array_equal(a, b)


@pytest.mark.parametrize("name,shape,extra,align", [
    ("quantize_jagged_rowwise", (37, 300), "offs1", 1),
    ("quantize_jagged_colwise", (300, 37), "offs0", 1),
    ("quantize_jagged_mx_rowwise", (37, 300), "offs1", 1),
    ("quantize_jagged_mx_colwise", (300, 37), "offs0", 1),
    ("quantize_mx_rowwise", (37, 256), None, 1),
    ("quantize_blockwise", (37, 256), (1, 128), 1),
    ("quantize_blockwise", (512, 256), (128, 128), 128),
    ("quantize_blockwise", (512, 40), (128, 1), 128),
    ("quantize_mx_3d_colwise", (7, 64, 24), None, 1),
])
def test_split_equals_whole(name, shape, extra, align):
    x = adversarial_bits(shape, 17)
    if extra == "offs1":
        args = (offsets_with_tail(shape[1], 5, 3),)
    elif extra == "offs0":
        args = (offsets_with_tail(shape[0], 5, 4),)
    elif extra is None:
        args = ()
    else:
        args = extra
    kw = {"canary": 0xA5} if "jagged" in name else {}
    whole = getattr(oracle, name)(x, *args, **kw)
    parts = oracle_pool.split_op(name, x, *args, align=align, parts=5, **kw)
    assert len(whole) == len(parts)
    for w, p in zip(whole, parts):
        assert same(w, p), name


@pytest.mark.parametrize("br,bc", [(128, 128), (1, 128), (128, 1)])
def test_blockwise_column_split_equals_whole(br, bc):
    x = adversarial_bits((256, 1024), 19)
    whole = oracle.quantize_blockwise(x, br, bc)
    parts = oracle_pool.split_op("quantize_blockwise", x, br, bc, align=bc, axis=1, parts=3)
    for w, p in zip(whole, parts):
        assert same(w, p)


def test_mx3d_experts_match_the_oracle():
    got = list(oracle_pool.mx3d_experts([0, 3], sweep=True, modes=("floor", "rceil"),
                                        shape=(64, 48)))
    assert [e for e, _, _ in got] == [0, 3]
    for e, bits, out in got:
        assert np.array_equal(bits, workloads.mx3d_sweep_expert(e, N=64, K=48))
        for mode in ("floor", "rceil"):
            q, s = oracle.quantize_mx_3d_colwise(bits[None], mode=mode)
            assert same(out[mode][0], q[0]) and same(out[mode][1], s[0])


def test_encode_matches_the_oracle():
    g = np.random.default_rng(4)
    y = (g.standard_normal(100_003) * 200).astype(np.float32)
    assert np.array_equal(oracle_pool.e4m3_encode(y), oracle.e4m3_encode(y))
