"""GPU parity on seeded random shapes: every dtype and epilogue, the automatic
plan and forced splits, prefetch depths and the general kernel, against the
oracle element by element.  Shapes are drawn so that most are ragged in M, N
and K (1..700) and some have several batches."""
import numpy as np
import pytest

import tiled_dense_gemm_mkl_amd as gm
from tiled_dense_gemm_mkl_amd import workloads
from gpu_helpers import TOL, assert_close, require_gpu, run_gemm

pytestmark = pytest.mark.gpu

DTYPES = ("f32", "f16", "bf16")
EPIS = ("identity", "relu", "silu")


def _cases(n=48, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = DTYPES[i % 3]
        epi = EPIS[(i // 3) % 3]
        M, N = (int(v) for v in rng.integers(1, 700, 2))
        # K a multiple of 8 elements (16-byte rows for 16-bit types) two times in three,
        # any K otherwise (the general kernel)
        K = int(rng.integers(1, 90)) * 8 if i % 3 else int(rng.integers(1, 700))
        L = int(rng.choice([1, 1, 2, 3]))
        mode = ("auto", "split", "depth", "general")[i % 4]
        out.append((i, dtype, epi, M, N, K, L, mode))
    return out


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"{c[0]}-{c[1]}-{c[2]}-{c[3]}x{c[4]}x{c[5]}x{c[6]}-{c[7]}")
def test_random_shape(orc, case):
    i, dtype, epi, M, N, K, L, mode = case
    A, B = workloads.random_operands(dtype, M, N, K, L, seed=1000 + i, dist_a=("normal", 1.0), dist_b=("normal", 1.0))
    kw = {}
    if mode == "split":
        kw = {"split_k": 1 + i % 4}
    elif mode == "depth":
        kw = {"prefetch_stages": i % 3}
    elif mode == "general":
        kw = {"force_general": True}
    try:
        C = run_gemm(A, B, dtype, epi, **kw)
    except gm.GemmMklError as e:
        # a forced split or depth that no configuration for this shape provides
        assert e.status == -6 and mode in ("split", "depth"), e
        C = run_gemm(A, B, dtype, epi)
    ref = orc.gemm64(A, B, dtype, epi)
    assert_close(C, ref, A, B, dtype, K, f"case {case}")
