"""CPU model of the data-parallel grid's workgroup -> tile mapping
(gemm_tile_kernel and xcd_block_raster in
tiled_dense_gemm_mkl_amd/csrc/gemm_kernels.hpp): every (batch, split, tile)
is covered exactly once, and with the XCD blocking each XCD (workgroup b runs
on XCD b % 8) covers one contiguous block of the tile grid."""
import pytest

from test_grouped_mapping import raster, xcd_remap


def tile_of(b, grid, tiles_m, tiles_n, L, split, group_m):
    t = xcd_remap(b, grid)
    tiles = tiles_m * tiles_n
    tile = t % tiles
    t //= tiles
    s, l = t % split, t // split
    if L == 1 and split == 1 and tiles_m % 2 == 0 and tiles_n % 4 == 0 and tiles >= 512:
        x, loc = b % 8, b // 8
        br, bc = tiles_m // 2, tiles_n // 4
        r, c = raster(loc, br, bc, group_m)
        return l, s, (x // 4) * br + r, (x % 4) * bc + c
    tm, tn = raster(tile, tiles_m, tiles_n, group_m)
    return l, s, tm, tn


@pytest.mark.parametrize("tiles_m,tiles_n,L,split", [
    (32, 32, 1, 1),     # 8192^3 in 256 x 256 tiles: blocked
    (16, 32, 1, 1),     # blocked, 8 x 8 blocks
    (2, 256, 1, 1),     # blocked, one tile row per block
    (4, 44, 1, 1),      # 176 tiles: one round, whole-grid raster
    (16, 16, 1, 1),     # 256 tiles: whole-grid raster
    (15, 32, 1, 1),     # odd tile rows: whole-grid raster
    (32, 30, 1, 1),     # columns not a multiple of 4
    (2, 14, 8, 1),      # batches
    (1, 32, 1, 4),      # split K
])
@pytest.mark.parametrize("group_m", [1, 4, 8])
def test_every_tile_once(tiles_m, tiles_n, L, split, group_m):
    gm_ = min(group_m, tiles_m)
    grid = tiles_m * tiles_n * L * split
    seen = [tile_of(b, grid, tiles_m, tiles_n, L, split, gm_) for b in range(grid)]
    assert sorted(seen) == sorted((l, s, m, n) for l in range(L) for s in range(split)
                                  for m in range(tiles_m) for n in range(tiles_n))


def test_blocked_xcd_reads_one_block():
    tiles_m = tiles_n = 32
    grid = tiles_m * tiles_n
    for x in range(8):
        cells = {tile_of(b, grid, tiles_m, tiles_n, 1, 1, 4)[2:] for b in range(x, grid, 8)}
        rows = {m for m, _ in cells}
        cols = {n for _, n in cells}
        assert len(rows) == 16 and len(cols) == 8 and len(cells) == 128
