"""Host check of the jagged colwise grid size: the number of work items per
column strip (long groups, and packs of up to 16 consecutive short groups
whose starts fall in one 1024-row block) must never exceed the bound the
library sizes its grid with, min(G, ext // 1010 + ext // 1024 + G // 16 + 1),
for any non-decreasing offsets.  Items are counted here the way the kernel
forms them; a bound that fell short would leave items without a workgroup
(their bytes and scales unwritten)."""
import numpy as np
import pytest

TROWS = 1024
PACK = 16


def count_items(offs, ext):
    """Long groups plus packs, by the kernel's rules."""
    G = len(offs)
    ends = np.clip(np.asarray(offs, dtype=np.int64), 0, ext)
    los = np.concatenate([[0], ends[:-1]])
    lng = (ends > los) & (ends - (los & ~15) > TROWS)
    items = int(lng.sum())
    run = -1
    for g in range(G):
        if g == 0 or lng[g] or lng[g - 1] or los[g] // TROWS != los[g - 1] // TROWS:
            run = g
        if not lng[g] and (g - run) % PACK == 0:
            items += 1
    return items


def bound(ext, G):
    return min(G, ext // (TROWS - 14) + ext // TROWS + G // PACK + 1)


def test_moe_and_uniform_cases():
    import workloads
    assert count_items(workloads.moe_offsets(), 16384) <= bound(16384, 8)
    for G in (1, 8, 32, 64, 128, 4096):
        offs = (np.arange(1, G + 1) * (16384 // G)).astype(np.int64)
        assert count_items(offs, 16384) <= bound(16384, G)


@pytest.mark.parametrize("seed", range(40))
def test_random_offsets(seed):
    g = np.random.default_rng(seed)
    ext = int(g.integers(0, 40000))
    G = int(g.choice([1, 2, 3, 7, 16, 33, 64, 100, 500, 4096]))
    mult = int(g.choice([1, 16]))
    # mixtures of long, short and empty groups
    cuts = np.sort(g.integers(0, ext // mult + 1, size=G)) * mult
    cuts[-1] = ext if g.random() < 0.7 else cuts[-1]
    cuts = np.maximum.accumulate(cuts)
    assert count_items(cuts, ext) <= bound(ext, G)


def test_worst_cases():
    # as many long groups as fit (1010 rows each, starting at 15 mod 16),
    # each followed by short groups spread over every block
    for ext in (1010, 5000, 16384, 100000):
        ends, e = [], 15
        while e + 1010 <= ext:
            ends += [e + 1010]
            e += 1010
            ends += [min(ext, e + k) for k in range(1, 40)]
        ends = np.maximum.accumulate(np.array(ends or [ext], dtype=np.int64))
        G = len(ends)
        assert count_items(ends, ext) <= bound(ext, G)
    # one short group starting in every block, and runs of exactly 16 + 1
    for ext in (4096, 65536):
        ends = np.arange(1, ext // TROWS + 1) * TROWS - 1
        assert count_items(ends, ext) <= bound(ext, len(ends))
        ends = np.repeat(np.arange(0, ext, 512), 17)[: 4096]
        ends = np.maximum.accumulate(ends)
        assert count_items(ends, ext) <= bound(ext, len(ends))
