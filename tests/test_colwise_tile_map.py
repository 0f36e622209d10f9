"""Host check of the colwise tile kernel's workgroup numbering, modelled on
the kernel's own integer steps: group g has max(1, ceil(s / CH)) chunks of
CH rows per 256-column tile, s being its rows from its start rounded down to
16 (0 for an empty group); workgroups run group by group, and within a group
in column blocks of B tiles (the largest B with B * nu <= 512, nu chunks per
tile), chunk-major inside a block.

Checked for random and adversarial offsets: every (group, column tile,
chunk) is taken by exactly one workgroup of the host's grid, tiles_c * (G +
(ext + 14 G) // CH); the chunks of one (group, column tile), which wait for
each other, lie in one block of at most 512 consecutive workgroup ids (so a
block fits among the workgroups resident at once); and a group's chunks
cover exactly its rows.  A numbering that broke any of these would leave
output unwritten or let an exchange wait on a workgroup that cannot start."""
import numpy as np
import pytest

SPAN = 512


def plan(offs, ext, cols, ch):
    ends = np.clip(np.asarray(offs, dtype=np.int64), 0, ext)
    los = np.concatenate([[0], ends[:-1]])
    his = np.maximum(ends, los)
    span = np.where(his > los, his - (los & ~15), 0)
    nu = np.where(span > ch, (span + ch - 1) // ch, 1)
    tiles_c = -(-cols // 256)
    G = len(offs)
    nblocks = tiles_c * (G + (ext + 14 * G) // ch)
    return los, his, nu, tiles_c, nblocks


def workgroup(b, nu, pre, tiles_c):
    """(group, column tile, chunk) of workgroup b, or None for a spare one."""
    j = b // tiles_c
    if j >= pre[-1]:
        return None
    g = int(np.searchsorted(pre[1:], j, side="right"))   # groups whose chunks all precede chunk j
    n = int(nu[g])
    local = b - int(pre[g]) * tiles_c
    B = max(1, min(SPAN // n, tiles_c))
    blk = local // (n * B)
    wb = min(B, tiles_c - blk * B)
    rr = local - blk * n * B
    k = rr // wb
    tc = blk * B + (rr - k * wb)
    return g, tc, k, blk


def check(offs, ext, cols, ch):
    los, his, nu, tiles_c, nblocks = plan(offs, ext, cols, ch)
    pre = np.concatenate([[0], np.cumsum(nu)])
    assert pre[-1] * tiles_c <= nblocks
    seen = {}
    for b in range(int(nblocks)):
        w = workgroup(b, nu, pre, tiles_c)
        if w is None:
            continue
        g, tc, k, blk = w
        assert 0 <= tc < tiles_c and 0 <= k < nu[g]
        assert (g, tc, k) not in seen
        seen[(g, tc, k)] = (b, blk)
    assert len(seen) == int(pre[-1]) * tiles_c
    blocks = {}
    for (g, tc, k), (b, blk) in seen.items():
        blocks.setdefault((g, blk), []).append(b)
    for ids in blocks.values():
        # a block is a run of consecutive workgroup ids, at most SPAN of them
        assert max(ids) - min(ids) + 1 == len(ids) <= SPAN
    for g in range(len(offs)):
        for tc in range(tiles_c):
            # the chunks of one (group, column tile) lie in one block
            assert len({seen[(g, tc, k)][1] for k in range(int(nu[g]))}) == 1
        # the chunks cover [lo, hi) exactly
        lo, hi = int(los[g]), int(his[g])
        rows = set()
        for k in range(int(nu[g])):
            a = (lo & ~15) + k * ch
            rows.update(range(max(a, lo), min(a + ch, hi)))
        assert rows == set(range(lo, hi))


@pytest.mark.parametrize("ch", [128, 256])
def test_moe_and_equal_groups(ch):
    import workloads
    check(workloads.moe_offsets(), 16384, 4096, ch)
    check(np.arange(1, 9) * 2048, 16384, 4096, ch)
    check(np.arange(1, 65) * 256, 16384, 520, ch)


@pytest.mark.parametrize("seed", range(30))
def test_random_offsets(seed):
    g = np.random.default_rng(9100 + seed)
    ext = int(g.integers(0, 20000))
    G = int(g.choice([1, 2, 3, 8, 17, 64, 65, 200, 256]))
    cols = 8 * int(g.integers(1, 700))
    mult = int(g.choice([1, 16]))
    cuts = np.sort(g.integers(0, ext // mult + 1, size=G)) * mult
    if g.random() < 0.7:
        cuts[-1] = ext
    check(np.maximum.accumulate(cuts), ext, cols, int(g.choice([128, 256])))


def test_long_groups_and_limits():
    # one group of the most chunks each chunk size allows, from an unaligned start
    check([15] * 255 + [255 * 128 - 15], 255 * 128 - 15, 264, 128)
    check([15] * 15 + [255 * 256 - 15], 255 * 256 - 15, 264, 256)
    # groups spanning just past a chunk from starts at 15 mod 16
    for L in (113, 114, 241, 242, 369):
        ends = np.arange(15 + L, 6000, L)
        check(np.concatenate([[15], ends]), 6000, 1032, 128)
        check(np.concatenate([[15], ends]), 6000, 1032, 256)
    # empty groups everywhere
    check([0, 0, 100, 100, 100, 5000, 5000], 5000, 256, 256)


@pytest.mark.parametrize("ch", [128, 256])
def test_most_chunks_per_row(ch):
    """Groups that each span one row more than a chunk from their 16-row-
    aligned start (two chunks for ch - 14 rows), each followed by a 14-row
    group that moves the next start back to 15 mod 16: about as many chunks
    per row as offsets can make."""
    ends, e = [], 15
    while len(ends) < 254:
        e += ch - 14                        # from a start at 15 mod 16: span ch + 1
        ends.append(e)
        e += 14                             # back to 15 mod 16
        ends.append(e)
    ext = ends[-1]
    los, his, nu, tiles_c, nblocks = plan(ends, ext, 256, ch)
    assert int(nu.sum()) == len(ends) + len(ends) // 2
    check(ends, ext, 256, ch)
