"""GPU results that follow from the definition alone, with no oracle call:

  - B = I (N = K): every output is one product a * 1, so C = epilogue(A)
    exactly (identity, ReLU), rounded once;
  - A = B = 1: every output is K, exact in fp32 partial sums, so C = epilogue(K)
    (the K of each workload shape is exactly representable in its dtype);
  - swapping A and B transposes C: bit for bit with integer inputs (every
    partial sum exact), within the tolerance with random inputs.
"""
import numpy as np
import pytest

import tiled_dense_gemm_mkl_amd as gm
from tiled_dense_gemm_mkl_amd import workloads
from gpu_helpers import TOL, assert_bits_equal, require_gpu, run_gemm, tol_error, widen_bits

pytestmark = pytest.mark.gpu

DTYPES = ("f32", "f16", "bf16")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _const(dtype, shape, v):
    return workloads.to_storage(np.full(shape, float(v)), dtype)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("K", [64, 264, 1024])
def test_identity_B_gives_epilogue_of_A(dtype, K):
    # normal values away from zero: no subnormal or signed-zero inputs
    x = np.random.default_rng(K).standard_normal((2, 150, K)) * 3.0
    A = workloads.to_storage(np.where(np.abs(x) < 1e-2, 1.0, x), dtype)
    B = workloads.to_storage(np.broadcast_to(np.eye(K), (2, K, K)), dtype)
    C = run_gemm(A, B, dtype, "identity")
    assert_bits_equal(C, A, f"{dtype} K={K} identity")
    R = run_gemm(A, B, dtype, "relu")
    Av = widen_bits(A, dtype)
    want = workloads.to_storage(np.where(Av > 0, Av, 0.0), dtype)   # exact: values of dtype and +0
    assert_bits_equal(R, want, f"{dtype} K={K} relu")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("K", [128, 2048, 8192, 18944])
def test_all_ones_gives_K(dtype, K):
    A = _const(dtype, (1, 96, K), 1.0)
    B = _const(dtype, (1, 80, K), 1.0)
    for epi in ("identity", "relu"):
        C = run_gemm(A, B, dtype, epi)
        assert_bits_equal(C, _const(dtype, (1, 96, 80), K), f"{dtype} K={K} {epi}")
    # SiLU(K) = K / (1 + e^-K) rounds to K for these K in every dtype
    C = run_gemm(A, B, dtype, "silu")
    assert_bits_equal(C, _const(dtype, (1, 96, 80), K), f"{dtype} K={K} silu")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", [(200, 136, 520, 1), (512, 5632, 2048, 1), (96, 300, 1000, 2)],
                         ids=lambda s: "x".join(map(str, s)))
def test_swapping_operands_transposes_C(dtype, shape):
    M, N, K, L = shape
    Ai, Bi = workloads.random_operands(dtype, M, N, K, L, seed=M + N, integer=True)
    C1 = run_gemm(Ai, Bi, dtype, "relu")
    C2 = run_gemm(Bi, Ai, dtype, "relu")
    assert_bits_equal(C2, np.ascontiguousarray(np.swapaxes(C1, 1, 2)), f"{dtype} {shape} integer")
    A, B = workloads.random_operands(dtype, M, N, K, L, seed=M + N + 1)
    C1 = run_gemm(A, B, dtype, "identity")
    C2 = run_gemm(B, A, dtype, "identity")
    ref = widen_bits(np.ascontiguousarray(np.swapaxes(C1, 1, 2)), dtype)
    err = tol_error(C2, ref, A, B, dtype, K)
    assert err <= TOL[dtype], f"{dtype} {shape}: swapped result differs by {err:.3e}"
