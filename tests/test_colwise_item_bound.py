"""Host check of the jagged colwise grid size: the number of work items per
column strip (long groups, and packs of up to 64 consecutive short groups
whose starts fall in one 1024-row block) must never exceed the bound the
library sizes its grid with, min(G, ext // 1010 + ext // 1024 + G // 64 + 1),
for any non-decreasing offsets.  With a workspace (split mode) a long group
of span n rows from its 16-row-aligned start makes ceil(n / 1536) items, and
the bound (with 512-row tiles, 4-wave workgroups) grows by
(ext + 15 * min(G, ext // 498)) // 1536; the workspace
holds one set per item number.  Items are counted here the way the kernel
forms them; a bound that fell short would leave items without a workgroup
(their bytes and scales unwritten).

The tile kernel (at most 256 groups; chunks of 128 rows x 256 columns for
groups of at most 128 rows on average and ext + 15 <= 255 * 128, else of 256
rows for at most 4096 rows per group on average and ext + 15 <= 255 * 256)
covers each group from its start rounded down to 16 rows: a group spanning
s rows that way has max(1, ceil(s / CH)) chunks per column tile, at most
G + (ext + 14 G) // CH in all, at most 255 each, and needs one workspace set
per column tile for every group spanning more than CH rows, at most
min(G, ext // (CH - 14)) groups; checked the same way."""
import numpy as np
import pytest

TROWS = 1024
PACK = 64


SPLIT_TROWS = 512             # 4-wave workgroups with a workspace
CHUNK = 3 * SPLIT_TROWS


def count_items(offs, ext, split=False):
    """Long groups (their chunks in split mode) plus packs, by the kernel's
    rules."""
    G = len(offs)
    tr = SPLIT_TROWS if split else TROWS
    ends = np.clip(np.asarray(offs, dtype=np.int64), 0, ext)
    los = np.concatenate([[0], ends[:-1]])
    lng = (ends > los) & (ends - (los & ~15) > tr)
    if split:
        span = ends - (los & ~15)
        items = int(np.where(lng, (span + CHUNK - 1) // CHUNK, 0).sum())
    else:
        items = int(lng.sum())
    run = -1
    for g in range(G):
        if g == 0 or lng[g] or lng[g - 1] or los[g] // tr != los[g - 1] // tr:
            run = g
        if not lng[g] and (g - run) % PACK == 0:
            items += 1
    return items


def bound(ext, G, split=False):
    tr = SPLIT_TROWS if split else TROWS
    b = min(G, ext // (tr - 14) + ext // tr + G // PACK + 1)
    if split:
        b += (ext + 15 * min(G, ext // (tr - 14))) // CHUNK
    return b


def check(offs, ext):
    check_tile(offs, ext)
    G = len(offs)
    assert count_items(offs, ext) <= bound(ext, G)
    assert count_items(offs, ext, True) <= bound(ext, G, True)


def test_split_chunks_fit_their_rows():
    """Every chunk of a long group holds at most CHUNK rows and the chunks
    cover the group: csz = round16(ceil(span / nc)), nc = ceil(span / CHUNK);
    the last chunk holds rows while nc < CHUNK / 16 (spans up to 96 chunks;
    a longer group's empty last chunk still takes part in the exchange)."""
    for span in list(range(SPLIT_TROWS + 1, 4 * CHUNK + 40)) + [16383, 16384, 100000, 196607]:
        nc = -(-span // CHUNK)
        csz = (-(-span // nc) + 15) // 16 * 16
        assert csz <= CHUNK and nc * csz >= span
        assert (nc - 1) * csz < span          # the last chunk holds rows


def tile_rows(ext, G):
    """Rows per chunk of the tile kernel for these extents, 0 if it does not
    apply."""
    if G > 256:
        return 0
    if ext <= 128 * G and ext + 15 <= 255 * 128:
        return 128
    if ext <= 4096 * G and ext + 15 <= 255 * 256:
        return 256
    return 0


def tile_counts(offs, ext, ch):
    """(chunks, groups of more than one chunk, most chunks of a group) by the
    tile kernel's rules: clamped ends, an empty group keeps one chunk."""
    ends = np.clip(np.asarray(offs, dtype=np.int64), 0, ext)
    los = np.concatenate([[0], ends[:-1]])
    span = np.where(ends > los, ends - (los & ~15), 0)
    chunks = np.where(span > ch, (span + ch - 1) // ch, 1)
    return int(chunks.sum()), int((span > ch).sum()), int(chunks.max(initial=1))


def check_tile(offs, ext):
    G = len(offs)
    for ch in (128, 256):
        chunks, nlong, most = tile_counts(offs, ext, ch)
        assert chunks <= G + (ext + 14 * G) // ch
        assert nlong <= min(G, ext // (ch - 14))
        if tile_rows(ext, G) == ch:
            assert most <= 255


def test_library_agrees_on_the_workspace_size():
    from mxfp8_quantization_moe_amd import _capi
    try:
        lib = _capi.load()
    except _capi.LibraryMissing:
        pytest.skip("library not built")
    cases = ((16384, 4096, 8), (1000, 64, 1), (65536, 8, 256), (0, 8, 3), (65280, 264, 16),
             (65281, 264, 16), (16384, 4096, 2), (16384, 4100, 4), (16384, 4096, 256),
             (32625, 264, 256), (32626, 264, 256), (65265, 264, 16), (65266, 264, 16))
    for ext, cols, G in cases:
        ch = tile_rows(ext, G)
        if ch:
            want = min(G, ext // (ch - 14)) * (-(-cols // 256)) * 264 * 4
        else:
            want = bound(ext, G, True) * (-(-cols // 64)) * 72 * 4
        assert lib.mxq_jagged_colwise_workspace_bytes(ext, cols, G) == want, (ext, cols, G)
    # more than 256 groups: the kernel without chunks, no workspace
    for G in (257, 4096):
        assert lib.mxq_jagged_colwise_workspace_bytes(65536, 8, G) == 0
    assert lib.mxq_jagged_colwise_workspace_bytes(-1, 8, 1) == -1
    assert lib.mxq_jagged_colwise_workspace_bytes(8, 8, 0) == -1


def test_moe_and_uniform_cases():
    import workloads
    check(workloads.moe_offsets(), 16384)
    for G in (1, 8, 32, 64, 128, 4096):
        offs = (np.arange(1, G + 1) * (16384 // G)).astype(np.int64)
        check(offs, 16384)


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
    check(cuts, ext)


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
        check(ends, ext)
    # one short group starting in every block, and runs of exactly one pack
    # plus one group (empty groups piled on one row)
    for ext in (4096, 65536):
        ends = np.arange(1, ext // TROWS + 1) * TROWS - 1
        check(ends, ext)
        ends = np.repeat(np.arange(0, ext, 512), PACK + 1)[: 4096]
        ends = np.maximum.accumulate(ends)
        check(ends, ext)
    # long groups whose spans each just exceed a chunk multiple, from a
    # start at 15 mod 16 (the most chunks per row)
    for ext in (20000, 100000):
        for L in (499, 513, 1010, 1537, 3073, 6145, 9217):
            ends = np.arange(15 + L, ext + 1, L, dtype=np.int64)
            if ends.size == 0:
                continue
            check(ends, ext)
