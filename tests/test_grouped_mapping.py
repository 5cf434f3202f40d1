"""CPU model of the grouped kernel's workgroup -> tile mapping
(gemm_grouped_kernel and find_group in
tiled_dense_gemm_mkl_amd/csrc/gemm_kernels.hpp), checked to cover every tile
of every group exactly once and nothing else.

The kernel launches (ceil(total_m / BM) + G) * tiles_n workgroups; workgroup
b takes id t = xcd_remap(b), row tile v = t / tiles_n of the concatenated
groups (offsets clamped to a non-decreasing sequence in [0, total_m]), finds
the group g holding v, and rasters the id inside that group.
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


def tiles_of_launch(offs, total_m, N, BM, BN, group_m):
    G = len(offs)
    tiles_n = (N + BN - 1) // BN
    row_tiles = (total_m + BM - 1) // BM + G
    grid = row_tiles * tiles_n
    seen = []
    for b in range(grid):
        t = xcd_remap(b, grid)
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
