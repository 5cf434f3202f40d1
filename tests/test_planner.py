"""CPU tests of the planner's choices (no GPU involved): the measured plans of
the named workloads, the two-workgroups-per-CU term of the 16-bit cost model,
and the opt-in 128 x 96 tile."""
import itertools

import pytest

import tiled_dense_gemm_mkl_amd as gm
from tiled_dense_gemm_mkl_amd import workloads

# plans measured best (or within timing noise) on MI355X for each workload
NAMED = {
    "bf16_512x5632x2048_relu": ("bf16 128x128 k64 waves2x2+4p mfma16", 3, 1),
    "f16_8192x8192x8192_identity": ("f16 256x256 k64 waves2x4 mfma32", 1, 1),
    "bf16_L8_512x3584x18944_silu": ("bf16 256x256 k32 waves2x2 mfma32", 4, 1),
    "f32_128x2048x2048_relu": ("f32 64x64 k32 waves2x2+4p mfma16", 3, 4),
    "f32_128x128x128_identity": ("f32 32x64 k32 waves1x2 mfma16", 2, 1),
}


def _plan(M, N, K, L, dtype, epi="relu", **kw):
    return gm.get_plan(M, N, K, L, gm.DTYPE_CODES[dtype], gm.EPILOGUE_CODES[epi], gm.make_opts(**kw) if kw else None)


@pytest.mark.parametrize("key", sorted(NAMED))
def test_named_workloads_keep_their_measured_plans(key):
    w = workloads.WORKLOADS[key]
    p = _plan(w.M, w.N, w.K, w.L, w.dtype, w.epilogue)
    assert (gm.config_names()[p["config_id"]], p["prefetch_stages"], p["split_k"]) == NAMED[key]


def test_grouped_workload_keeps_its_configuration():
    """4096 rows in 8 groups x 5632 x 2048 bf16, measured with the empty row
    blocks of each group's last tile skipped: 256 x 256 tiles with 8 waves
    105 us, with 4 waves 115 us, 128 x 128 + 4 producers 132 us."""
    cid = gm.grouped_config(8, 4096, 5632, 2048, gm.BF16, gm.EPI_RELU)
    assert gm.config_names()[cid] == "bf16 256x256 k64 waves2x4 mfma32"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("M,N", [(256, 5632), (256, 8192), (512, 3584)])
def test_short_K_mid_grids_run_two_workgroups_per_CU(dtype, M, N):
    """257..512 tiles of 64 x 64 with K = 512 (8 chunks): two depth-3 rings
    (64 KB each) fit in a CU's LDS, so all tiles run at once; measured 5.5-5.8
    against 6.7-6.9 us for 128 x 128 tiles."""
    p = _plan(M, N, 512, 1, dtype)
    tiles = -(-M // 64) * -(-N // 64)
    assert 256 < tiles <= 512
    assert gm.config_names()[p["config_id"]] == f"{dtype} 64x64 k64 waves2x2 mfma32"
    assert (p["prefetch_stages"], p["split_k"]) == (3, 1)


def test_fp32_two_workgroups_per_CU_only_where_measured_faster():
    """fp32's weaker factor: 128 x 2048 x 2048 keeps 4 splits (256 units;
    8 splits measured slower), while 1024 x 1024 x 4096 (256 tiles of 64 x 64)
    splits in 2 so that two workgroups share each CU (72.7 against 78.4 us)."""
    assert _plan(128, 2048, 2048, 1, "f32")["split_k"] == 4
    p = _plan(1024, 1024, 4096, 1, "f32")
    assert gm.config_names()[p["config_id"]] == "f32 64x64 k32 waves2x2+4p mfma16" and p["split_k"] == 2


@pytest.mark.parametrize("M,N,K", [(128, 2048, 2048), (512, 2048, 2048), (1024, 1024, 4096), (128, 4096, 4096),
                                   (256, 1024, 1024), (2048, 2048, 2048), (1000, 1100, 520), (4096, 4096, 4096)])
def test_fp32_takes_the_64x64_tile_with_producer_waves(M, N, K):
    """The 64 x 64 fp32 tile with four producer waves measured fastest on every
    fp32 shape tried (128 x 2048 x 2048 S=4 with the fix-up 13.2-13.6 us against
    14.9-15.3 without producers; 4096^3 985 against 1029 us on 128 x 128)."""
    p = _plan(M, N, K, 1, "f32")
    assert gm.config_names()[p["config_id"]] == "f32 64x64 k32 waves2x2+4p mfma16"


def test_opt_in_tile_is_never_chosen_but_can_be_forced():
    names = gm.config_names()
    for dtype in ("bf16", "f16"):
        for M, N, K in itertools.product((1, 256, 512, 1024, 4096), (96, 1024, 3584, 5632, 8192), (64, 512, 2048, 8192)):
            p = _plan(M, N, K, 1, dtype)
            assert "128x96" not in names[p["config_id"]], (dtype, M, N, K)
        cid = names.index(f"{dtype} 128x96 k64 waves2x2+4p mfma16")
        p = _plan(512, 5632, 2048, 1, dtype, config_id=cid)
        assert p["config_id"] == cid and p["prefetch_stages"] == 4
        assert p["grid"] == 4 * 59   # 5632 / 96 = 58.7 column tiles


@pytest.mark.parametrize("G,rows,want", [
    (8, 4096, "bf16 256x256 k64 waves2x4 mfma32"),    # 667 us against 826 on 128 x 128 + producers
    (32, 2048, "bf16 256x256 k64 waves2x4 mfma32"),   # 1503 against 1795
    (64, 64, "bf16 128x128 k64 waves2x2+4p mfma32"),  # 361 against 385 on 256 x 256
])
def test_grouped_tile_follows_group_size(G, rows, want):
    cid = gm.grouped_config(G, G * rows, 5632, 2048, gm.BF16, gm.EPI_RELU)
    assert gm.config_names()[cid] == want


# bf16 shapes of the planner audit (graph replay, one box) whose automatic plan
# changed with the 64 x 64 producer tile, the 128 x 256 producer tile's figure
# and the rule that 16-bit plans take the in-kernel fix-up only when forced
AUDITED = {
    (1024, 1024, 4096): ("bf16 64x64 k64 waves2x2+4p mfma16", 1),      # 15.6 us; 32 x 32 MFMAs 17.2-17.6 (four fix-up pieces of 128 x 128: 22.7)
    (256, 4096, 4096): ("bf16 64x64 k64 waves2x2+4p mfma16", 1),       # 32 x 32 MFMAs 17.3 us (22.7)
    (512, 2048, 2048): ("bf16 64x64 k64 waves2x2+4p mfma16", 1),       # 9.2 us (32 x 32 MFMAs 9.5, no producers 10.7)
    (128, 5632, 2048): ("bf16 64x64 k64 waves2x2+4p mfma16", 1),       # 32 x 32 MFMAs 9.3 us (9.8)
    (1024, 8192, 8192): ("bf16 128x256 k64 waves2x2+4p mfma16", 1),    # 101.8 us; 32 x 32 MFMAs 109-112 (two fix-up pieces of 256 x 256: 131.7)
    (1024, 8192, 2048): ("bf16 128x256 k64 waves2x2+4p mfma16", 1),    # 31.0 us; 32 x 32 MFMAs 32.2 (256 x 128: 37.5)
    (4096, 8192, 2048): ("bf16 256x256 k64 waves2x4 mfma32", 1),       # 116-118 us (128 x 256: 124.2)
    (256, 5632, 512): ("bf16 64x64 k64 waves2x2 mfma32", 1),           # two per CU: 5.70 us (with producers 5.89)
}


@pytest.mark.parametrize("shape", sorted(AUDITED))
def test_audited_bf16_plans(shape):
    p = _plan(*shape, 1, "bf16")
    assert (gm.config_names()[p["config_id"]], p["split_k"]) == AUDITED[shape]
    assert p["fixup"] == 0


def test_16bit_fixup_only_when_forced():
    """The in-kernel fix-up is never chosen automatically for 16-bit types
    (no shape measured it faster than the best plan without it), but a forced
    split or a forced fix-up still takes it."""
    for M, N, K in [(256, 8192, 2048), (1024, 8192, 8192), (1024, 1024, 4096), (512, 3584, 18944)]:
        assert _plan(M, N, K, 1, "bf16")["fixup"] == 0
    assert _plan(512, 5632, 2048, 1, "bf16", split_k=2, fixup=True)["fixup"] == 1
    assert _plan(512, 5632, 2048, 1, "bf16", split_k=2)["fixup"] == 1


def test_long_rows_stay_inside_one_buffer_descriptor():
    """A tile kernel addresses a tile's rows of A and B through one buffer
    descriptor whose offsets are below 2^31: for every K the plan's tile must
    span fewer bytes than that (with a row of slack), a forced configuration
    that would not is NOT_AVAILABLE, and rows too long for every tile take the
    general kernel, which indexes with 64-bit pointers, without repacking."""
    names = gm.config_names()
    for dtype, es in ((gm.BF16, 2), (gm.F32, 4)):
        for K in (2 ** 20, 2 ** 21, 2 ** 22, 2 ** 23, 2 ** 24, 2 ** 26, 2 ** 26 + 1, 2 ** 30 + 3):
            p = gm.get_plan(512, 512, K, 1, dtype, gm.EPI_RELU)
            if p["general"]:
                assert p["packed"] == 0 and p["split_k"] == 1
                continue
            assert (max(p["block_m"], p["block_n"]) + 1) * K * es < 2 ** 31, (dtype, K, p)
        for cid, name in enumerate(names):
            if not name.startswith("bf16" if dtype == gm.BF16 else "f32"):
                continue
            bm, bn = (int(x) for x in name.split()[1].split("x"))
            span = (max(bm, bn) + 1) * es
            # the tile's rows just below 2^31 bytes: the forced configuration runs
            K = (2 ** 31 - 65536) // span // 64 * 64
            assert gm.get_plan(512, 512, K, 1, dtype, gm.EPI_RELU, gm.make_opts(config_id=cid))["config_id"] == cid
            K = 2 ** 31 // span // 64 * 64 + 64   # just past: refused
            with pytest.raises(gm.GemmMklError) as e:
                gm.get_plan(512, 512, K, 1, dtype, gm.EPI_RELU, gm.make_opts(config_id=cid))
            assert e.value.status == -6, (name, K)
    # the largest K is planned on the general kernel, never packed
    assert gm.get_plan(4, 4, 2 ** 30 + 3, 1, gm.BF16, gm.EPI_IDENTITY)["general"] == 1


def test_grouped_long_rows_fit_one_descriptor_or_are_refused():
    """The grouped kernels address a tile's rows the same way: the chosen
    configuration's tile spans less than 2^31 bytes of rows, and rows too long
    for every grouped configuration are NOT_AVAILABLE (there is no general
    grouped kernel) rather than planned past the range."""
    names = gm.config_names()
    for K in (2 ** 20, 2 ** 22, 2 ** 23):
        cid = gm.grouped_config(4, 512, 256, K, gm.BF16, gm.EPI_RELU)
        bm, bn = (int(x) for x in names[cid].split()[1].split("x"))
        assert (max(bm, bn) + 1) * K * 2 < 2 ** 31, (K, names[cid])
    with pytest.raises(gm.GemmMklError) as e:
        gm.grouped_config(4, 512, 256, 2 ** 25, gm.BF16, gm.EPI_RELU)
    assert e.value.status == -6
