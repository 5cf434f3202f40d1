"""GPU parity of the persistent grid (one workgroup per compute unit, one
prefetch ring across each workgroup's tiles).

Every tile is computed exactly as by the data-parallel grid of the same
configuration and depth (same chunks in the same order, same MFMA sequence,
same epilogue), so the two must agree bit for bit; the persistent results are
also checked against the oracle (sampled entries, integer inputs bit-exact).
"""
import pytest

import tiled_dense_gemm_mkl_amd as gm
from tiled_dense_gemm_mkl_amd import workloads
from gpu_helpers import TOL, assert_bits_equal, require_gpu, run_gemm, sample_indices, tol_error

pytestmark = pytest.mark.gpu

CONFIG = "{} 128x128 k64 waves2x2+4p mfma32"
SHAPES = [
    (1000, 1100, 520, 1),      # fewer tiles than CUs (forced), ragged M, N and K
    (1030, 900, 264, 3),       # batches, ragged
    (2000, 2100, 1000, 2),     # 544 tiles: two full rounds and a partial one
    (1024, 1024, 64, 1),       # one chunk per tile
    (700, 2200, 40, 1),        # one ragged chunk per tile
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _cid(dtype):
    return gm.config_names().index(CONFIG.format(dtype))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_persistent_equals_data_parallel(dtype, shape):
    M, N, K, L = shape
    cid = _cid(dtype)
    A, B = workloads.random_operands(dtype, M, N, K, L, seed=M + K)
    for epi in ("identity", "relu", "silu"):
        plan = gm.get_plan(M, N, K, L, gm.DTYPE_CODES[dtype], gm.EPILOGUE_CODES[epi],
                           gm.make_opts(config_id=cid, persistent=True))
        assert plan["persistent"] == 1
        Cp = run_gemm(A, B, dtype, epi, config_id=cid, persistent=True)
        Cd = run_gemm(A, B, dtype, epi, config_id=cid, prefetch_stages=plan["prefetch_stages"], split_k=1,
                      persistent=False)
        assert_bits_equal(Cp, Cd, f"{dtype} {shape} {epi}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_persistent_against_oracle(orc, dtype):
    M, N, K, L = 2000, 2100, 1000, 2
    cid = _cid(dtype)
    A, B = workloads.random_operands(dtype, M, N, K, L, seed=11, dist_a=("normal", 1.0), dist_b=("normal", 0.02))
    C = run_gemm(A, B, dtype, "relu", config_id=cid, persistent=True)
    li, mi, ni = sample_indices(L, M, N, 3000, seed=12)
    ref = orc.gemm_entries64(A, B, dtype, "relu", li, mi, ni)
    err = tol_error(C[li, mi, ni], ref, A, B, dtype, K)
    assert err <= TOL[dtype], f"err {err:.3e}"
    Ai, Bi = workloads.random_operands(dtype, M, N, K, L, seed=13, integer=True)
    Ci = run_gemm(Ai, Bi, dtype, "identity", config_id=cid, persistent=True)
    refi = orc.round_to_dtype(orc.gemm_entries64(Ai, Bi, dtype, "identity", li, mi, ni), dtype)
    assert_bits_equal(Ci[li, mi, ni], refi, "integer sample")


def test_persistent_many_rounds_deterministic(orc):
    """4096 x 5632 x 2048 bf16 (1408 tiles of 128 x 128, five and a half
    rounds on 256 workgroups): two runs agree bit for bit, and sampled
    entries meet the tolerance."""
    M, N, K = 4096, 5632, 2048
    cid = _cid("bf16")
    plan = gm.get_plan(M, N, K, 1, gm.BF16, gm.EPI_RELU, gm.make_opts(config_id=cid, persistent=True))
    assert plan["persistent"] == 1 and plan["grid"] == 256
    A, B = workloads.random_operands("bf16", M, N, K, 1, seed=21, dist_a=("normal", 1.0), dist_b=("normal", 0.02))
    C1 = run_gemm(A, B, "bf16", "relu", config_id=cid, persistent=True)
    C2 = run_gemm(A, B, "bf16", "relu", config_id=cid, persistent=True)
    assert_bits_equal(C1, C2, "run to run")
    li, mi, ni = sample_indices(1, M, N, 2000, seed=22)
    ref = orc.gemm_entries64(A, B, "bf16", "relu", li, mi, ni)
    assert tol_error(C1[li, mi, ni], ref, A, B, "bf16", K) <= TOL["bf16"]
