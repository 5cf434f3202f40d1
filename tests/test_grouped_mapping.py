"""CPU model of the grouped kernel's workgroup -> tile mapping
(gemm_grouped_kernel and find_group in
tiled_dense_gemm_mkl_amd/csrc/gemm_kernels.hpp), checked to cover every tile
of every group exactly once and nothing else.

The kernel launches (ceil(total_m / BM) + G) * tiles_n workgroups.  With at
most 512 groups each workgroup first counts the T tiles that exist, and
workgroup b (on XCD x = b % 8) takes id t = x * (T // 8) + min(x, T % 8) + b // 8
when b // 8 is below that XCD's share (T // 8, one more for the first T % 8
XCDs); with more groups t = xcd_remap(b).  Row tile v = t / tiles_n of the
concatenated groups (offsets clamped to a non-decreasing sequence in
[0, total_m]) gives the group g holding v, and the id inside that group is
rastered.  A group's last row tile computes only the MF-row blocks that hold
rows, shared out over the wave rows (run_live).
"""
import numpy as np
import pytest


def xcd_remap(wg, grid, xcd=8):
    per = grid // xcd
    full = per * xcd
    if wg >= full:
        return wg
    return (wg % xcd) * per + wg // xcd


def raster(tile, tiles_m, tiles_n, group_m):
    width = group_m * tiles_n
    first_m = (tile // width) * group_m
    gsize = min(tiles_m - first_m, group_m)
    return first_m + (tile % width) % gsize, (tile % width) // gsize


def find_group(offs, total_m, v, BM):
    """(g, tile of v inside g, first row, rows) or g = -1 past the last tile."""
    ends = np.maximum.accumulate(np.clip(np.asarray(offs, np.int64), 0, total_m))
    starts = np.concatenate([[0], ends[:-1]])
    before = 0
    for g, (s, e) in enumerate(zip(starts, ends)):
        nt = (e - s + BM - 1) // BM
        if before <= v < before + nt:
            return g, v - before, int(s), int(e - s)
        before += nt
    return -1, 0, 0, 0


EXACT_SCAN = 512   # kGroupedExactScan


def total_row_tiles(offs, total_m, BM):
    ends = np.maximum.accumulate(np.clip(np.asarray(offs, np.int64), 0, total_m))
    starts = np.concatenate([[0], ends[:-1]])
    return int(sum((e - s + BM - 1) // BM for s, e in zip(starts, ends)))


def tile_id(b, grid, G, total):
    """Workgroup b -> tile id t, or None for a workgroup that exits at once."""
    if G <= EXACT_SCAN:
        x, j = b & 7, b >> 3
        q, rem = total >> 3, total & 7
        if j >= q + (1 if x < rem else 0):
            return None
        return x * q + min(x, rem) + j
    return xcd_remap(b, grid)


def tiles_of_launch(offs, total_m, N, BM, BN, group_m, xcd_of=None):
    G = len(offs)
    tiles_n = (N + BN - 1) // BN
    row_tiles = (total_m + BM - 1) // BM + G
    grid = row_tiles * tiles_n
    total = total_row_tiles(offs, total_m, BM) * tiles_n
    seen = []
    for b in range(grid):
        t = tile_id(b, grid, G, total)
        if t is None:
            continue
        assert G > EXACT_SCAN or t < total
        if xcd_of is not None:
            xcd_of[b % 8] = xcd_of.get(b % 8, 0) + 1
        v = t // tiles_n
        g, tv, row0, rows = find_group(offs, total_m, v, BM)
        if g < 0:
            continue
        rg = (rows + BM - 1) // BM
        u = t - (v - tv) * tiles_n
        assert 0 <= u < rg * tiles_n
        tm, tn = raster(u, rg, tiles_n, group_m)
        assert 0 <= tm < rg and 0 <= tn < tiles_n
        seen.append((g, tm, tn))
    return seen


def expected_tiles(offs, total_m, N, BM, BN):
    ends = np.maximum.accumulate(np.clip(np.asarray(offs, np.int64), 0, total_m))
    starts = np.concatenate([[0], ends[:-1]])
    tiles_n = (N + BN - 1) // BN
    return sorted((g, tm, tn) for g, (s, e) in enumerate(zip(starts, ends))
                  for tm in range((e - s + BM - 1) // BM) for tn in range(tiles_n))


CASES = [
    ([612, 2689, 2895, 3045, 3219, 3430, 3765, 4096], 4096, 5632),   # the 8-group workload's ends
    ([0, 5, 305, 306, 434, 434, 563, 627], 630, 200),                  # empty, one-row, ragged groups
    ([1] * 9, 12, 96),
    ([50, 20, 120, 400, -5, 180], 200, 96),                            # offsets to be clamped
    ([517], 517, 1000),
    (list(range(1, 601)), 600, 64),                                    # past the exact scan: remap over the grid
]


@pytest.mark.parametrize("offs,total_m,N", CASES)
@pytest.mark.parametrize("BM,BN", [(128, 128), (256, 256), (64, 64)])
@pytest.mark.parametrize("group_m", [1, 4, 8])
def test_every_tile_exactly_once(offs, total_m, N, BM, BN, group_m):
    seen = tiles_of_launch(offs, total_m, N, BM, BN, group_m)
    assert sorted(seen) == expected_tiles(offs, total_m, N, BM, BN)


def test_group_major_order_keeps_a_group_together():
    """Within one XCD's share of ids, a group's tiles are consecutive: the
    ids of group g are exactly [S_g * tiles_n, (S_g + R_g) * tiles_n)."""
    offs, total_m, N, BM, BN = CASES[0][0], 4096, 5632, 128, 128
    tiles_n = (N + BN - 1) // BN
    grid = ((total_m + BM - 1) // BM + len(offs)) * tiles_n
    by_group = {}
    for t in range(grid):
        g = find_group(offs, total_m, t // tiles_n, BM)[0]
        if g >= 0:
            by_group.setdefault(g, []).append(t)
    for g, ids in by_group.items():
        assert ids == list(range(ids[0], ids[0] + len(ids))), f"group {g} not contiguous"


@pytest.mark.parametrize("offs,total_m,N", CASES[:5])
@pytest.mark.parametrize("BM,BN", [(128, 128), (256, 256)])
def test_xcds_get_equal_shares_of_the_tiles(offs, total_m, N, BM, BN):
    """With the exact count every XCD gets T // 8 or T // 8 + 1 tiles (the
    empty ids at the end of the grid no longer all land on the last XCDs)."""
    per = {}
    tiles_of_launch(offs, total_m, N, BM, BN, 4, xcd_of=per)
    total = total_row_tiles(offs, total_m, BM) * ((N + BN - 1) // BN)
    counts = [per.get(x, 0) for x in range(8)]
    assert sum(counts) == total
    assert max(counts) - min(counts) <= 1


def live_blocks(live, BM, MF, waves_m):
    """The MF-row blocks the waves compute for a tile with `live` rows: wave
    row wm computes fragment rows i < fml, i.e. blocks i * waves_m + wm."""
    FM = BM // waves_m // MF
    blocks = (live + MF - 1) // MF
    done = []
    for wm in range(waves_m):
        fml = min(max(-(-(blocks - wm) // waves_m), 0), FM)
        done += [i * waves_m + wm for i in range(fml)]
    return sorted(done), FM


@pytest.mark.parametrize("BM,MF,waves_m", [(256, 32, 2), (128, 32, 2), (64, 32, 2), (256, 16, 4), (128, 16, 2)])
def test_live_row_blocks_cover_every_row_once(BM, MF, waves_m):
    for live in range(1, BM + 1):
        done, FM = live_blocks(live, BM, MF, waves_m)
        assert done == list(range((live + MF - 1) // MF)), (live, done)
        # the wave rows' shares differ by at most one fragment row
        fmls = [sum(1 for b in done if b % waves_m == wm) for wm in range(waves_m)]
        assert max(fmls) - min(fmls) <= 1 and max(fmls) <= FM


def test_grouped_workload_mfma_work_within_five_percent():
    """The 8-group bf16 workload (ends below) on 128- and 256-row tiles: the
    rows the MFMAs compute exceed the 4096 real rows by about 3%, against
    12.5% and 25% when every partly filled tile is computed in full."""
    ends = [612, 2689, 2895, 3045, 3219, 3430, 3765, 4096]
    sizes = np.diff([0] + ends)
    for BM in (128, 256):
        rows = 0
        for m in sizes:
            full, tail = divmod(int(m), BM)
            rows += full * BM + (-(-tail // 32) * 32)
        assert rows <= 1.05 * 4096, (BM, rows)
