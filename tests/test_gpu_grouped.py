"""GPU parity of the grouped GEMM (gemm_mkl_grouped) against the CPU oracle.

Group g owns rows [offs[g-1], offs[g]) of A and C and its own B[g]; rows in no
group must be left untouched.  Random inputs meet the same tolerance as the
dense path; integer-valued inputs are bit-exact for identity and ReLU.
"""
import numpy as np
import pytest

import tiled_dense_gemm_mkl_amd as gm
from tiled_dense_gemm_mkl_amd import workloads
from gpu_helpers import TOL, assert_bits_equal, require_gpu, tol_error, widen_bits

pytestmark = pytest.mark.gpu

DTYPES = ("f32", "f16", "bf16")
SENTINEL = {"f32": np.float32(-7.0), "f16": np.uint16(0xC700), "bf16": np.uint16(0xC0E0)}   # -7 in each dtype


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _configs_of(dtype):
    """Every configuration of dtype (those without grouped kernels answer NOT_AVAILABLE)."""
    return [cid for cid, name in enumerate(gm.config_names()) if name.split()[0] == dtype]


def _operands(dtype, total_m, G, N, K, seed, integer=False):
    A, _ = workloads.random_operands(dtype, total_m, 1, K, 1, seed, integer=integer)
    _, B = workloads.random_operands(dtype, 1, N, K, G, seed + 1, integer=integer)
    return A[0], B


def _run(A, B, offs, dtype, epilogue, **kw):
    import torch

    a = workloads.storage_to_torch(np.ascontiguousarray(A), dtype).cuda()
    b = workloads.storage_to_torch(np.ascontiguousarray(B), dtype).cuda()
    o = torch.from_numpy(np.ascontiguousarray(offs, dtype=np.int32)).cuda()
    out_bits = np.full((A.shape[0], B.shape[1]), SENTINEL[dtype])
    out = workloads.storage_to_torch(out_bits, dtype).cuda()
    c = gm.gemm_grouped(a, b, o, epilogue, out=out, **kw)
    torch.cuda.synchronize()
    return workloads.torch_to_storage(c)


def _check(C, ref64, A, B, dtype, K, what):
    covered = ~np.isnan(ref64[:, 0]) if ref64.size else np.zeros(0, bool)
    # rows in no group: untouched
    assert np.all(C[~covered] == SENTINEL[dtype]), f"{what}: rows outside every group were written"
    if covered.any():
        got = widen_bits(C[covered], dtype)
        assert np.all(np.isfinite(got)), f"{what}: non-finite output"
        err = tol_error(C[covered], ref64[covered], A, B, dtype, K)
        assert err <= TOL[dtype], f"{what}: err {err:.3e} > {TOL[dtype]:.0e}"


SIZES = [
    [0, 5, 300, 1, 128, 0, 129, 64],      # empty groups, one row, exact and ragged tiles
    [517],                                 # one group
    [1] * 9,                               # many one-row groups
]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("sizes", SIZES, ids=["mixed", "single", "ones"])
def test_grouped_parity_all_epilogues(orc, dtype, sizes):
    N, K = 200, 264 if dtype != "f32" else 132
    G = len(sizes)
    offs = np.cumsum(sizes).astype(np.int32)
    total_m = int(offs[-1]) + 3                       # 3 trailing rows in no group
    A, B = _operands(dtype, total_m, G, N, K, seed=77)
    for epi in ("identity", "relu", "silu"):
        ref = orc.gemm_grouped64(A, B, offs, dtype, epi)
        C = _run(A, B, offs, dtype, epi)
        _check(C, ref, A, B, dtype, K, f"{dtype} {epi} sizes={sizes}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_grouped_every_config_and_integer_bit_exact(orc, dtype):
    sizes = [37, 0, 260, 3, 129]
    offs = np.cumsum(sizes).astype(np.int32)
    total_m, G, N, K = int(offs[-1]), len(sizes), 190, 512
    A, B = _operands(dtype, total_m, G, N, K, seed=5)
    Ai, Bi = _operands(dtype, total_m, G, N, K, seed=6, integer=True)
    ref = orc.gemm_grouped64(A, B, offs, dtype, "relu")
    refi = orc.round_to_dtype(orc.gemm_grouped64(Ai, Bi, offs, dtype, "identity"), dtype)
    ran = 0
    for cid in _configs_of(dtype):
        try:
            C = _run(A, B, offs, dtype, "relu", config_id=cid)
        except gm.GemmMklError as e:
            assert e.status == -6          # a configuration without grouped kernels
            continue
        ran += 1
        _check(C, ref, A, B, dtype, K, f"config {cid}")
        Ci = _run(Ai, Bi, offs, dtype, "identity", config_id=cid)
        assert_bits_equal(Ci, refi, f"integer config {cid}")
    assert ran >= 1


def test_grouped_offsets_are_clamped(orc):
    """Decreasing or out-of-range offsets never address rows outside A or C:
    the kernels use the running maximum of the offsets clamped to [0, total_m]."""
    dtype, N, K = "bf16", 96, 128
    total_m = 200
    raw = np.array([50, 20, 120, 400, -5, 180], np.int32)
    A, B = _operands(dtype, total_m, len(raw), N, K, seed=9)
    clamped = np.maximum.accumulate(np.clip(raw, 0, total_m)).astype(np.int32)
    ref = orc.gemm_grouped64(A, B, clamped, dtype, "identity")
    C = _run(A, B, raw, dtype, "identity")
    _check(C, ref, A, B, dtype, K, "clamped offsets")


def test_grouped_deterministic_and_matches_dense_for_one_group(orc):
    import torch

    dtype, M, N, K = "f16", 333, 250, 640
    A, B = _operands(dtype, M, 1, N, K, seed=3)
    offs = np.array([M], np.int32)
    C1 = _run(A, B, offs, dtype, "silu")
    C2 = _run(A, B, offs, dtype, "silu")
    assert_bits_equal(C1, C2, "run to run")
    ref = orc.gemm_grouped64(A, B, offs, dtype, "silu")
    _check(C1, ref, A, B, dtype, K, "one group")


def test_grouped_workload_parity(orc):
    """The grouped workload bench.py times, in the launch configuration it
    times, against the oracle on 48 sampled rows (every column of each; 16 of
    them also with integer inputs, bit-exact)."""
    w = workloads.GROUPED_WORKLOADS["grouped_bf16_G8_4096x5632x2048_relu"]
    A, B, offs = workloads.make_grouped_inputs(w)
    rows = np.random.default_rng(0).choice(w.total_m, 48, replace=False)
    C = _run(A, B, offs, w.dtype, w.epilogue)
    # sampled rows through the oracle (a row's group comes from the offsets)
    groups = np.searchsorted(offs, rows, side="right")
    for r, g in zip(rows, groups):
        ref = orc.gemm_grouped64(A[r:r + 1], B[g:g + 1], np.array([1], np.int32), w.dtype, w.epilogue)
        err = tol_error(C[r:r + 1], ref, A, B, w.dtype, w.K)
        assert err <= TOL[w.dtype], f"row {r} (group {g}): err {err:.3e}"
    Ai, Bi, _ = workloads.make_grouped_inputs(w, integer=True)
    Ci = _run(Ai, Bi, offs, w.dtype, "relu")
    for r, g in zip(rows[:16], groups[:16]):
        refi = orc.round_to_dtype(orc.gemm_grouped64(Ai[r:r + 1], Bi[g:g + 1], np.array([1], np.int32),
                                                     w.dtype, "relu"), w.dtype)
        assert_bits_equal(Ci[r:r + 1], refi, f"integer row {r}")


@pytest.mark.parametrize("dtype,epilogue", [("bf16", "silu"), ("f16", "relu")])
def test_grouped_large_groups_parity(orc, dtype, epilogue):
    """8 groups of 4096 rows (N = K = 2048): the automatic choice is the
    256 x 256 tile with 2 x 4 waves at depth 1.  Checked against the oracle on
    40 sampled rows, among them the first and last row of every group (every
    column of each), and bit-exact on 16 of them with integer inputs."""
    G, rows_per, N, K = 8, 4096, 2048, 2048
    total_m = G * rows_per
    cid = gm.grouped_config(G, total_m, N, K, gm.DTYPE_CODES[dtype], gm.EPILOGUE_CODES[epilogue])
    assert gm.config_names()[cid] == f"{dtype} 256x256 k64 waves2x4 mfma32"
    offs = np.arange(1, G + 1, dtype=np.int32) * rows_per
    A, B = _operands(dtype, total_m, G, N, K, seed=77)
    edges = np.concatenate([offs - rows_per, offs - 1])
    rows = np.concatenate([edges, np.random.default_rng(1).choice(total_m, 40 - edges.size, replace=False)])
    C = _run(A, B, offs, dtype, epilogue)
    groups = np.searchsorted(offs, rows, side="right")
    for r, g in zip(rows, groups):
        ref = orc.gemm_grouped64(A[r:r + 1], B[g:g + 1], np.array([1], np.int32), dtype, epilogue)
        err = tol_error(C[r:r + 1], ref, A, B, dtype, K)
        assert err <= TOL[dtype], f"row {r} (group {g}): err {err:.3e}"
    Ai, Bi = _operands(dtype, total_m, G, N, K, seed=78, integer=True)
    Ci = _run(Ai, Bi, offs, dtype, "identity")
    for r, g in zip(rows[:16], groups[:16]):
        refi = orc.round_to_dtype(orc.gemm_grouped64(Ai[r:r + 1], Bi[g:g + 1], np.array([1], np.int32),
                                                     dtype, "identity"), dtype)
        assert_bits_equal(Ci[r:r + 1], refi, f"integer row {r}")


def test_grouped_empty_problems_launch_nothing():
    for args in [(0, 8, 8, 64), (3, 0, 8, 64), (3, 8, 0, 64)]:
        G, total_m, N, K = args
        assert gm.gemm_mkl_grouped(None, None, None, None, G, total_m, N, K, gm.BF16, gm.EPI_RELU, None, None) == 0


def _cid(name):
    return gm.config_names().index(name)


@pytest.mark.parametrize("cfg", ["bf16 256x256 k64 waves2x4 mfma32", "bf16 256x256 k32 waves2x2 mfma32",
                                 "bf16 128x128 k64 waves2x2+4p mfma32", "bf16 64x64 k64 waves2x2 mfma32"])
def test_grouped_last_tile_every_live_block_count(orc, cfg):
    """A group's last tile computes only its row blocks that hold rows, shared
    out over the wave rows: groups whose last tile holds 1..8 blocks of 32
    rows (and one more row than a block boundary, or one fewer) run through
    every such count, bit for bit on integer inputs, within the tolerance on
    random ones; rows of no group stay untouched."""
    dtype = "bf16"
    sizes = [32 * b - 1 for b in range(1, 9)] + [256 + 32 * b + 1 for b in range(0, 8)] + [512]
    offs = np.cumsum(sizes).astype(np.int32)
    total_m, G, N, K = int(offs[-1]) + 5, len(sizes), 136, 256
    A, B = _operands(dtype, total_m, G, N, K, seed=21)
    Ai, Bi = _operands(dtype, total_m, G, N, K, seed=22, integer=True)
    cid = _cid(cfg)
    C = _run(A, B, offs, dtype, "relu", config_id=cid)
    _check(C, orc.gemm_grouped64(A, B, offs, dtype, "relu"), A, B, dtype, K, cfg)
    Ci = _run(Ai, Bi, offs, dtype, "relu", config_id=cid)
    refi = orc.round_to_dtype(orc.gemm_grouped64(Ai, Bi, offs, dtype, "relu"), dtype)
    covered = ~np.isnan(orc.gemm_grouped64(Ai, Bi, offs, dtype, "relu")[:, 0])
    assert_bits_equal(Ci[covered], refi[covered], f"integer {cfg}")


def test_grouped_many_groups_take_the_remapped_grid(orc):
    """More than 512 groups: the workgroups skip the exact tile count and map
    their ids over the whole grid instead (ids past the last tile exit)."""
    dtype = "bf16"
    rng = np.random.default_rng(31)
    sizes = rng.integers(0, 9, size=700)
    offs = np.cumsum(sizes).astype(np.int32)
    total_m, G, N, K = int(offs[-1]), len(sizes), 72, 64
    A, B = _operands(dtype, total_m, G, N, K, seed=32)
    C = _run(A, B, offs, dtype, "identity")
    _check(C, orc.gemm_grouped64(A, B, offs, dtype, "identity"), A, B, dtype, K, "700 groups")
    Ai, Bi = _operands(dtype, total_m, G, N, K, seed=33, integer=True)
    refi = orc.round_to_dtype(orc.gemm_grouped64(Ai, Bi, offs, dtype, "identity"), dtype)
    assert_bits_equal(_run(Ai, Bi, offs, dtype, "identity"), refi, "700 groups integer")


@pytest.mark.parametrize("dtype", DTYPES)
def test_grouped_special_values(orc, dtype):
    """+inf, -inf and NaN planted in A rows of three groups (one of them a
    one-row group) and in the last k of one column of a fourth group's B, on
    integer inputs: NaN exactly where the oracle has NaN, every other output
    of the grouped rows bit for bit, rows in no group untouched."""
    sizes = [0, 37, 130, 1, 64]
    G, N, K = len(sizes), 96, 136
    offs = np.cumsum(sizes).astype(np.int32)
    total_m = int(offs[-1]) + 2
    A, B = _operands(dtype, total_m, G, N, K, seed=91, integer=True)
    Av, Bv = widen_bits(A, dtype), widen_bits(B, dtype)
    Av[3, 0] = np.inf                 # group 1
    Av[40, 100] = -np.inf             # group 2
    Av[167, 5] = np.nan               # group 3, its only row
    Bv[4, 17, K - 1] = np.inf         # group 4, column 17
    A, B = workloads.to_storage(Av, dtype), workloads.to_storage(Bv, dtype)
    rows = np.arange(total_m) < offs[-1]
    for epi in ("identity", "relu"):
        C = _run(A, B, offs, dtype, epi)
        assert np.all(C[~rows] == SENTINEL[dtype]), f"{dtype} {epi}: rows outside every group were written"
        want64 = orc.gemm_grouped64(A, B, offs, dtype, epi)[rows]
        got = widen_bits(C[rows], dtype)
        assert np.array_equal(np.isnan(got), np.isnan(want64)), f"{dtype} {epi}: NaN pattern"
        num = ~np.isnan(want64)
        assert_bits_equal(C[rows][num], orc.round_to_dtype(want64, dtype)[num], f"{dtype} {epi}")
        assert np.isinf(want64).any() and (epi == "relu" or np.isnan(want64).any())
