"""Special values through the GEMM on the GPU, against the oracle: infinite and
NaN inputs, sums past the output type's range, and subnormal inputs and
outputs.

The inputs are built so that every fp32 partial sum the GPU forms is exact
wherever the result is finite (small integers, or powers of two of one sign
per row), so the GPU's result must equal the oracle's single rounding bit for
bit; NaN is compared as a pattern, since its payload and sign are not
specified.  IEEE arithmetic fixes the outcomes the oracle computes in binary64:
an infinite product dominates every finite term, inf * 0 and inf - inf are
NaN, and ReLU maps NaN and -inf to +0 (where(x > 0, x, 0)).

Every case runs through the automatic plan, two K splits (summed inside the
kernel where the plan has a fix-up kernel, and by the reduction kernel), the
general kernel, and stream-K where the dtype has a stream-K configuration.
"""
from __future__ import annotations

import numpy as np
import pytest

import tiled_dense_gemm_mkl_amd as gm
from tiled_dense_gemm_mkl_amd import workloads
from gpu_helpers import TOL, assert_bits_equal, require_gpu, run_gemm, widen_bits

pytestmark = pytest.mark.gpu

DTYPES = ("f32", "f16", "bf16")
PLANS = {
    "auto": {},
    "split2": {"split_k": 2},
    "split2-reduce": {"split_k": 2, "fixup": False},
    "general": {"force_general": True},
    "streamk": {"streamk": True},
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _bits(v: np.ndarray, dtype: str) -> np.ndarray:
    return workloads.to_storage(v, dtype)


def _run(A, B, dtype, epi, plan):
    try:
        return run_gemm(A, B, dtype, epi, **PLANS[plan])
    except gm.GemmMklError as e:
        if plan == "streamk" and e.status == -6:
            pytest.skip(f"no stream-K configuration for {dtype}")
        raise


def _compare(C, orc, A, B, dtype, epi, what):
    """Bit for bit where the oracle's result is a number, NaN where it is NaN."""
    ref64 = orc.gemm64(A, B, dtype, epi)
    ref = orc.round_to_dtype(ref64, dtype)
    got = widen_bits(C, dtype)
    want = widen_bits(ref, dtype)
    assert np.array_equal(np.isnan(got), np.isnan(want)), f"{what}: NaN pattern differs"
    num = ~np.isnan(want)
    assert_bits_equal(C[num], ref[num], what)
    return want


@pytest.mark.parametrize("plan", sorted(PLANS))
@pytest.mark.parametrize("epi", ("identity", "relu"))
@pytest.mark.parametrize("dtype", DTYPES)
def test_infinite_and_nan_inputs(orc, dtype, epi, plan):
    """Integers in [-2, 2] with +inf, -inf and NaN planted in A and B: rows and
    columns that meet them come out infinite or NaN exactly as in binary64."""
    M, N, K, L = 70, 45, 200, 2
    rng = np.random.default_rng(4100)
    Av = rng.integers(-2, 3, size=(L, M, K)).astype(np.float64)
    Bv = rng.integers(-2, 3, size=(L, N, K)).astype(np.float64)
    Av[0, 3, 5] = np.inf                      # one infinite term
    Av[0, 7, 150] = -np.inf                   # in the ragged last chunk
    Av[1, 11, 20] = np.nan
    Av[1, 13, 1], Av[1, 13, 2] = np.inf, -np.inf   # inf - inf wherever both meet non-zero B
    Bv[0, 4, 30] = np.inf                     # a whole column of infinities (NaN where A is 0)
    Bv[1, 44, 199] = np.nan                   # the last column, the last k
    A, B = _bits(Av, dtype), _bits(Bv, dtype)
    C = _run(A, B, dtype, epi, plan)
    want = _compare(C, orc, A, B, dtype, epi, f"{dtype} {epi} {plan}")
    if epi == "identity":
        assert np.isinf(want).sum() > 0 and np.isnan(want).sum() > 0   # the case is what it claims
    else:
        assert not np.isnan(want).any() and np.isinf(want).sum() > 0


@pytest.mark.parametrize("plan", sorted(PLANS))
@pytest.mark.parametrize("dtype", DTYPES)
def test_sums_past_the_output_range_round_to_infinity(orc, dtype, plan):
    """Sums at and beyond the largest finite output value: the GPU's rounding
    of the fp32 sum must overflow to +-inf exactly where the oracle's does.

    fp16: A in {0, +-1} (one sign per row), B integers in [0, 2048], K = 128:
    sums up to 2^18, exact in fp32, about half of them past 65520 (the tie
    above 65504, which rounds to inf).
    bf16 and fp32: A in {0, +-2^120} (one sign per row, few non-zeros), B in
    {0, 2^6, 2^7}: terms of 2^126 or 2^127 of one sign per row, so every
    partial sum is a multiple of 2^126 and exact until it reaches 2^128,
    which overflows fp32 as it overflows both output types."""
    M, N, L = 66, 40, 1
    K = 128 if dtype == "f16" else 64
    rng = np.random.default_rng(4200)
    sign = np.where(rng.integers(0, 2, size=(L, M, 1)) == 1, 1.0, -1.0)
    if dtype == "f16":
        Av = rng.integers(0, 2, size=(L, M, K)).astype(np.float64) * sign
        Bv = rng.integers(0, 2049, size=(L, N, K)).astype(np.float64)
    else:
        Av = np.where(rng.random((L, M, K)) < 0.05, 2.0 ** 120, 0.0) * sign
        Bv = rng.choice([0.0, 2.0 ** 6, 2.0 ** 7], size=(L, N, K))
    A, B = _bits(Av, dtype), _bits(Bv, dtype)
    C = _run(A, B, dtype, "identity", plan)
    want = _compare(C, orc, A, B, dtype, "identity", f"{dtype} {plan}")
    fin = np.isfinite(want)
    assert (~fin).sum() > 0 and fin.sum() > 0 and (want[fin] != 0).sum() > 0


def _pow2(rng, shape, exps):
    """Powers of two 2^e, e drawn from exps, with random signs."""
    e = rng.choice(exps, size=shape)
    return np.ldexp(np.where(rng.integers(0, 2, size=shape) == 1, 1.0, -1.0), e)


# (A exponents, B exponents): subnormal inputs whose products are normal fp32,
# and normal inputs whose products and sums are subnormal in the output type
SUBNORMAL_IN = {"f32": ([-140, -145], [20, 22]), "f16": ([-20, -22], [8, 10]), "bf16": ([-130, -132], [10, 12])}
SUBNORMAL_OUT = {"f32": ([-70, -72], [-70, -71]), "f16": ([-12, -13], [-10, -11]), "bf16": ([-68, -70], [-62, -64])}


@pytest.mark.parametrize("plan", sorted(PLANS))
@pytest.mark.parametrize("case", ("subnormal inputs", "subnormal outputs"))
@pytest.mark.parametrize("dtype", DTYPES)
def test_subnormals(orc, dtype, case, plan):
    """Gradual underflow on both sides of the products.  The terms are 48
    signed powers of two spread over at most eight binades, so every fp32
    partial sum is exact (subnormal ones included) and the result must equal
    the oracle's single rounding bit for bit."""
    M, N, K, L = 33, 40, 48, 1
    rng = np.random.default_rng(4300 + DTYPES.index(dtype))
    ea, eb = (SUBNORMAL_IN if case == "subnormal inputs" else SUBNORMAL_OUT)[dtype]
    Av, Bv = _pow2(rng, (L, M, K), ea), _pow2(rng, (L, N, K), eb)
    A, B = _bits(Av, dtype), _bits(Bv, dtype)
    # the inputs are what the case says: exactly representable, and subnormal where claimed
    assert np.array_equal(widen_bits(A, dtype), Av) and np.array_equal(widen_bits(B, dtype), Bv)
    C = _run(A, B, dtype, "identity", plan)
    want = _compare(C, orc, A, B, dtype, "identity", f"{dtype} {case} {plan}")
    tiny = {"f32": 2.0 ** -126, "f16": 2.0 ** -14, "bf16": 2.0 ** -126}[dtype]
    if case == "subnormal inputs":
        assert np.all(np.abs(Av) < tiny)
    else:
        assert np.any((want != 0) & (np.abs(want) < tiny))


@pytest.mark.parametrize("dtype", DTYPES)
def test_silu_of_infinities(orc, dtype):
    """SiLU on sums that are +inf, -inf and NaN: +inf stays +inf; -inf gives
    -inf / inf = NaN on both sides; finite sums stay within the tolerance."""
    M, N, K, L = 40, 36, 72, 1
    rng = np.random.default_rng(4400)
    Av = rng.integers(-2, 3, size=(L, M, K)).astype(np.float64)
    Bv = rng.integers(1, 3, size=(L, N, K)).astype(np.float64)   # positive: sign of an infinite row kept
    Av[0, 2, 9] = np.inf
    Av[0, 5, 9] = -np.inf
    Av[0, 8, 40] = np.nan
    A, B = _bits(Av, dtype), _bits(Bv, dtype)
    C = run_gemm(A, B, dtype, "silu")
    got = widen_bits(C, dtype)
    want = orc.gemm64(A, B, dtype, "silu")
    assert np.array_equal(np.isnan(got), np.isnan(want)), "NaN pattern"
    assert np.all(got[np.isinf(want)] == want[np.isinf(want)])
    assert np.all(got[0, 2] == np.inf) and np.all(np.isnan(got[0, 5])) and np.all(np.isnan(got[0, 8]))
    fin = np.isfinite(want)
    err = np.max(np.abs(got[fin] - want[fin])) / (K * 2 * 2)
    assert err <= TOL[dtype], f"finite entries: err {err:.3e}"
