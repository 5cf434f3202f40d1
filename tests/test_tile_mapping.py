"""CPU model of the data-parallel grid's workgroup -> tile mapping
(TileMap / map_workgroup in tiled_dense_gemm_mkl_amd/csrc/gemm_kernels.hpp),
written with plain integer division: every (batch, split, tile) is covered
exactly once, and with the XCD blocking each XCD (workgroup b runs on XCD
b % 8) covers one contiguous block of the tile grid.  The library's own map
(multiply-high divisions, gemm_mkl_tile_order) must equal the model."""
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


# ------------------------------------------------------------------ the library's own map

import math  # noqa: E402

import tiled_dense_gemm_mkl_amd as gm  # noqa: E402


@pytest.mark.parametrize("M,N,K,L,dtype,split", [
    (512, 5632, 2048, 1, "bf16", None),      # 236 tiles of 128 x 96, one round
    (8192, 8192, 8192, 1, "f16", None),      # blocked
    (4096, 8192, 2048, 1, "bf16", None),     # blocked
    (4096, 5632, 2048, 1, "bf16", None),
    (512, 3584, 18944, 8, "bf16", None),     # batches
    (700, 2200, 264, 3, "f16", None),        # ragged last raster group, batches
    (1000, 1100, 520, 1, "f32", None),
    (128, 2048, 2048, 1, "f32", None),
    (300, 5000, 4096, 2, "bf16", 3),         # forced K split with batches
    (2000, 2100, 1000, 2, "bf16", 2),
    (96, 80, 18944, 1, "bf16", 7),
    (1, 1, 8, 1, "bf16", None),
    (4224, 4352, 64, 1, "f16", None),        # blocked, group rows past the block
])
def test_library_map_matches_the_model(M, N, K, L, dtype, split):
    """gemm_mkl_tile_order runs the kernel's own map (multiply-high divisions,
    built by the host) for every workgroup of the planned grid; it must equal
    the model above, written with plain integer division."""
    code = gm.DTYPE_CODES[dtype]
    # (the in-kernel fix-up has a map of its own, tested below)
    opts = gm.make_opts(split_k=split, fixup=False)
    plan = gm.get_plan(M, N, K, L, code, gm.EPI_RELU, opts)
    if plan["general"] or plan["streamk"] or plan["persistent"]:
        with pytest.raises(gm.GemmMklError):
            gm.tile_order(M, N, K, L, code, gm.EPI_RELU, opts)
        return
    tiles_m, tiles_n = math.ceil(M / plan["block_m"]), math.ceil(N / plan["block_n"])
    S, grid = plan["split_k"], plan["grid"]
    assert grid == tiles_m * tiles_n * L * S
    got = gm.tile_order(M, N, K, L, code, gm.EPI_RELU, opts)
    want = [tile_of(b, grid, tiles_m, tiles_n, L, S, min(4, tiles_m)) for b in range(grid)]
    assert got.shape == (grid, 4)
    assert [tuple(r) for r in got.tolist()] == want


def test_library_map_refuses_short_output_and_other_grids():
    code = gm.BF16
    with pytest.raises(gm.GemmMklError):
        gm.tile_order(8192, 8192, 64, 1, code, gm.EPI_RELU, gm.make_opts(force_general=True))
    lib = gm.load()
    import numpy as np
    grid = gm.get_plan(512, 5632, 2048, 1, code, gm.EPI_RELU)["grid"]
    out = np.zeros(4 * (grid - 1), np.int32)
    assert lib.gemm_mkl_tile_order(512, 5632, 2048, 1, code, gm.EPI_RELU, None, out.ctypes.data, out.size) == -1
    assert lib.gemm_mkl_tile_order(512, 5632, 2048, 1, code, gm.EPI_RELU, None, None, 4 * grid) == -1
    out = np.zeros(4 * grid, np.int32)
    assert lib.gemm_mkl_tile_order(512, 5632, 2048, 1, code, gm.EPI_RELU, None, out.ctypes.data, out.size) == 0
    assert lib.gemm_mkl_tile_order(0, 5632, 2048, 1, code, gm.EPI_RELU, None, None, 0) == 0


@pytest.mark.parametrize("M,N,K,L,dtype,S,cfg", [
    (512, 5632, 2048, 1, "bf16", 2, "bf16 128x192 k64 waves2x2+4p mfma32"),   # 120 tiles, 240 workgroups
    (512, 5632, 2048, 1, "bf16", 3, "bf16 128x192 k64 waves2x2+4p mfma32"),
    (128, 2048, 2048, 1, "f32", 4, "f32 64x64 k32 waves2x2 mfma16"),          # 64 tiles, 4 pieces each
    (300, 700, 1000, 3, "f16", 2, "f16 128x128 k64 waves2x2+4p mfma32"),      # ragged, batches
    (512, 3584, 18944, 8, "bf16", 2, "bf16 256x256 k32 waves2x2 mfma32"),     # 224 tiles
    (100, 100, 4096, 1, "bf16", 6, "bf16 128x128 k64 waves2x2+4p mfma32"),    # one tile, six pieces
])
def test_fixup_grid_places_every_piece_of_a_tile_on_one_xcd(M, N, K, L, dtype, S, cfg):
    """Split-K with the in-kernel fix-up: every (batch, piece, tile) is held by
    exactly one workgroup, the S pieces of a tile share one XCD (workgroup b
    runs on XCD b % 8, so their L2), and each XCD's tiles are a contiguous run
    of the [batch][raster] order of at most ceil(tiles / 8) tiles."""
    import tiled_dense_gemm_mkl_amd as gm

    names = gm.config_names()
    code = gm.DTYPE_CODES[dtype]
    o = gm.make_opts(split_k=S, config_id=names.index(cfg), fixup=True)
    plan = gm.get_plan(M, N, K, L, code, gm.EPI_RELU, o)
    assert plan["fixup"] == 1 and plan["split_k"] == S
    tm_, tn_ = -(-M // plan["block_m"]), -(-N // plan["block_n"])
    T = tm_ * tn_ * L
    per = -(-T // 8)
    assert plan["grid"] == per * 8 * S
    assert plan["counter_bytes"] == -(-T * 128 // 256) * 256   # one 128-byte line per tile
    assert plan["workspace_bytes"] == plan["counter_bytes"] + T * S * plan["block_m"] * plan["block_n"] * 4
    order = gm.tile_order(M, N, K, L, code, gm.EPI_RELU, o)
    seen = {}
    xcd_of_tile = {}
    for b, (l, s, tm, tn) in enumerate(order.tolist()):
        if l < 0:
            assert (l, s, tm, tn) == (-1, -1, -1, -1)
            continue
        assert 0 <= l < L and 0 <= s < S and 0 <= tm < tm_ and 0 <= tn < tn_
        key = (l, s, tm, tn)
        assert key not in seen, f"{key} held twice"
        seen[key] = b
        xcd_of_tile.setdefault((l, tm, tn), set()).add(b % 8)
    assert len(seen) == T * S
    assert all(len(x) == 1 for x in xcd_of_tile.values()), "pieces of one tile on different XCDs"
    # each XCD holds at most `per` tiles
    count = {}
    for (l, tm, tn), xs in xcd_of_tile.items():
        x = next(iter(xs))
        count[x] = count.get(x, 0) + 1
    assert max(count.values()) <= per


def test_fixup_plan_options():
    import tiled_dense_gemm_mkl_amd as gm

    names = gm.config_names()
    # a configuration without fix-up kernels, forced with a split: not available
    cid = names.index("bf16 256x128 k64 waves4x2 mfma32")
    with pytest.raises(gm.GemmMklError) as e:
        gm.get_plan(512, 5632, 2048, 1, gm.BF16, gm.EPI_RELU, gm.make_opts(split_k=2, config_id=cid, fixup=True))
    assert e.value.status == -6
    # more than six pieces: not available with the fix-up
    cid = names.index("bf16 128x192 k64 waves2x2+4p mfma32")
    with pytest.raises(gm.GemmMklError):
        gm.get_plan(512, 5632, 2048, 1, gm.BF16, gm.EPI_RELU, gm.make_opts(split_k=8, config_id=cid, fixup=True))
    # both flags at once are invalid
    with pytest.raises(gm.GemmMklError) as e:
        o = gm.make_opts(fixup=True)
        o.flags |= gm._binding.OPT_NO_FIXUP
        gm.get_plan(512, 5632, 2048, 1, gm.BF16, gm.EPI_RELU, o)
    assert e.value.status == -1
    # GEMM_MKL_OPT_NO_FIXUP keeps the reduction kernel for a forced split
    p = gm.get_plan(512, 5632, 2048, 1, gm.BF16, gm.EPI_RELU, gm.make_opts(split_k=2, config_id=cid, fixup=False))
    assert p["fixup"] == 0 and p["split_k"] == 2
    # the fp32 128 x 2048 x 2048 workload: four splits summed in the kernel
    # (measured 15.1 against 16.0 us per call with the reduction kernel)
    p = gm.get_plan(128, 2048, 2048, 1, gm.F32, gm.EPI_RELU)
    assert p["fixup"] == 1 and p["split_k"] == 4


@pytest.mark.parametrize("M,N,K,L,dtype", [(1000, 1100, 520, 1, "bf16"), (300, 200, 4096, 3, "f32")])
def test_streamk_counters_one_line_per_tile(M, N, K, L, dtype):
    """Stream-K keeps one counter per tile of all batches, each on its own
    128-byte line (32 ints apart), followed by two partial tiles per workgroup."""
    import tiled_dense_gemm_mkl_amd as gm

    plan = gm.get_plan(M, N, K, L, gm.DTYPE_CODES[dtype], gm.EPI_RELU, gm.make_opts(streamk=True))
    assert plan["streamk"] == 1
    T = -(-M // plan["block_m"]) * -(-N // plan["block_n"]) * L
    assert plan["counter_bytes"] == -(-T * 128 // 256) * 256
    assert plan["workspace_bytes"] == plan["counter_bytes"] + 2 * plan["grid"] * plan["block_m"] * plan["block_n"] * 4
