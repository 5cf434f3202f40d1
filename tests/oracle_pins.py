"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``check_*`` function takes a loaded oracle library handle and raises
AssertionError when the oracle disagrees with:
  - exact rational arithmetic (``fractions.Fraction``) on tiny GEMMs,
  - closed forms (identity B gives C = epilogue(A); all-ones gives C = K),
  - numpy's binary64 matmul and conversions, torch's exact bf16 widening,
  - the IEEE round-to-nearest-even definition at constructed midpoints,
  - high-precision SiLU and RMSNorm from mpmath, torch's own binary64 RMSNorm,
    closed forms and invariants of the RMSNorm.

The functions are shared by ``test_oracle.py`` (they must pass on the real
oracle) and by the planted-mistake test (each mutant must fail one of them).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

import oracle

DTYPES = ("f32", "f16", "bf16")
EPIS = ("identity", "relu", "silu")


# ------------------------------------------------------------------ helpers

def _random_bits(rng, dtype, shape, scale=1.0):
    """Random finite values of dtype as stored bits (drawn here, not by the oracle)."""
    x = rng.standard_normal(size=shape) * scale
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    # bf16: truncate a float32 pattern (any bf16 value is a valid input)
    return (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _exact_values(bits, dtype):
    """Exact rational value of every stored element, independent of the oracle."""
    if dtype == "f32":
        vals = bits.astype(np.float64)
    elif dtype == "f16":
        vals = bits.view(np.float16).astype(np.float64)
    else:
        vals = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return vals


def _frac_gemm(Av, Bv):
    L, M, K = Av.shape
    N = Bv.shape[1]
    out = [[[Fraction(0)] * N for _ in range(M)] for _ in range(L)]
    mag = [[[Fraction(0)] * N for _ in range(M)] for _ in range(L)]
    for l in range(L):
        for m in range(M):
            for n in range(N):
                s = Fraction(0)
                a = Fraction(0)
                for k in range(K):
                    p = Fraction(float(Av[l, m, k])) * Fraction(float(Bv[l, n, k]))
                    s += p
                    a += abs(p)
                out[l][m][n] = s
                mag[l][m][n] = a
    return out, mag


def _silu_mp(x):
    import mpmath

    mpmath.mp.prec = 200
    xv = mpmath.mpf(x) if not isinstance(x, Fraction) else mpmath.mpf(x.numerator) / x.denominator
    return float(xv / (1 + mpmath.exp(-xv)))


def _relu_exact(x):
    return x if x > 0 else 0


# ------------------------------------------------------------------ conversions

def check_widen_f16_exhaustive(lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.widen(bits, "f16", lib)
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "f16 widen: NaN pattern"
    assert np.array_equal(got[~nan], want[~nan]), "f16 widen differs from numpy"
    # sign of zero
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan])), "f16 widen: sign"


def check_widen_bf16_exhaustive(lib):
    import torch

    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.widen(bits, "bf16", lib)
    want = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "bf16 widen: NaN pattern"
    assert np.array_equal(got[~nan], want[~nan]), "bf16 widen differs from torch"


def _consecutive_midpoints(vals):
    """For sorted finite positive values v: midpoints (v_i + v_{i+1}) / 2 (exact in fp64)."""
    lo, hi = vals[:-1], vals[1:]
    return lo, hi, (lo + hi) / 2.0


def check_round_bf16_midpoints(lib):
    # every finite positive bf16 value, ascending (bit patterns 0x0000 .. 0x7f7f)
    pos_bits = np.arange(0, 0x7F80, dtype=np.uint32)
    vals = (pos_bits << 16).view(np.float32).astype(np.float64)
    # values are fixed points of the rounding
    got = oracle.round_to_dtype(vals, "bf16", lib)
    assert np.array_equal(got.astype(np.uint32), pos_bits), "bf16 rounding moves exact values"
    got = oracle.round_to_dtype(-vals[1:], "bf16", lib)
    assert np.array_equal(got.astype(np.uint32), pos_bits[1:] | 0x8000), "bf16 negative values"
    lo, hi, mid = _consecutive_midpoints(vals)
    lo_b, hi_b = pos_bits[:-1], pos_bits[1:]
    even = np.where(lo_b % 2 == 0, lo_b, hi_b)
    got = oracle.round_to_dtype(mid, "bf16", lib).astype(np.uint32)
    assert np.array_equal(got, even), "bf16 ties must go to even"
    up = np.nextafter(mid, np.inf)
    dn = np.nextafter(mid, -np.inf)
    assert np.array_equal(oracle.round_to_dtype(up, "bf16", lib).astype(np.uint32), hi_b), "bf16 above midpoint"
    assert np.array_equal(oracle.round_to_dtype(dn, "bf16", lib).astype(np.uint32), lo_b), "bf16 below midpoint"
    # overflow: the midpoint between the largest finite value and 2^128 is a tie -> inf
    big = float((2 - 2.0 ** -7) * 2.0 ** 127)
    edge = float((2 - 2.0 ** -8) * 2.0 ** 127)
    got = oracle.round_to_dtype(np.array([big, np.nextafter(edge, 0), edge, -edge]), "bf16", lib)
    assert list(got) == [0x7F7F, 0x7F7F, 0x7F80, 0xFF80], "bf16 overflow threshold"
    # a value that double rounding through binary32 gets wrong
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert int(oracle.round_to_dtype(np.array([x]), "bf16", lib)[0]) == 0x3F81, "bf16 single rounding"


def check_round_f16_vs_numpy(lib):
    rng = np.random.default_rng(7)
    # random magnitudes over the whole fp16 range, subnormals and overflow included
    x = np.ldexp(rng.uniform(1.0, 2.0, 200000), rng.integers(-30, 18, 200000))
    x *= np.where(rng.integers(0, 2, x.size) == 1, -1.0, 1.0)
    want = x.astype(np.float16).view(np.uint16)
    got = oracle.round_to_dtype(x, "f16", lib)
    assert np.array_equal(got, want), "f16 rounding differs from numpy on random values"
    # midpoints between consecutive fp16 values, and one binary64 ulp to each side
    pos_bits = np.arange(0, 0x7C00, dtype=np.uint16)
    vals = pos_bits.view(np.float16).astype(np.float64)
    lo, hi, mid = _consecutive_midpoints(vals)
    for probe in (mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)):
        want = probe.astype(np.float16).view(np.uint16)
        got = oracle.round_to_dtype(probe, "f16", lib)
        assert np.array_equal(got, want), "f16 rounding differs from numpy near midpoints"
    lo_b = pos_bits[:-1].astype(np.uint32)
    hi_b = pos_bits[1:].astype(np.uint32)
    even = np.where(lo_b % 2 == 0, lo_b, hi_b)
    assert np.array_equal(oracle.round_to_dtype(mid, "f16", lib).astype(np.uint32), even), "f16 ties to even"


def check_round_f32_vs_cast(lib):
    rng = np.random.default_rng(8)
    x = np.ldexp(rng.uniform(1.0, 2.0, 200000), rng.integers(-160, 129, 200000))
    x *= np.where(rng.integers(0, 2, x.size) == 1, -1.0, 1.0)
    with np.errstate(over="ignore"):
        want = x.astype(np.float32)
    got = oracle.round_to_dtype(x, "f32", lib)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), "f32 rounding differs from the binary32 cast"


# ------------------------------------------------------------------ epilogues

def check_epilogue_values(lib):
    ep = lambda x, e: oracle.epilogue64(x, e, lib)  # noqa: E731
    for x in (-3.5, -1e-300, 0.0, 2.0 ** -1074, 1.0, 7.25, 1e300):
        assert ep(x, "identity") == x
        assert ep(x, "relu") == max(x, 0.0)
    assert math.copysign(1.0, ep(-0.0, "relu")) == 1.0, "relu(-0) must be +0 (where(x > 0, x, 0))"
    assert ep(0.0, "silu") == 0.0
    assert ep(1.0, "silu") == 1.0 / (1.0 + math.exp(-1.0))
    assert ep(1000.0, "silu") == 1000.0
    v = ep(-1000.0, "silu")
    assert v == 0.0 and math.copysign(1.0, v) == -1.0, "silu(-1000) is -0"
    rng = np.random.default_rng(9)
    for x in np.concatenate([rng.uniform(-40, 40, 300), rng.uniform(-1e-3, 1e-3, 50)]):
        s = ep(float(x), "silu")
        ref = _silu_mp(float(x))
        assert abs(s - ref) <= 4 * np.spacing(abs(ref)) + 1e-300, f"silu({x}) = {s}, want {ref}"
        # odd-part identity silu(x) - silu(-x) = x
        d = s - ep(float(-x), "silu")
        assert abs(d - x) <= 8 * np.spacing(max(abs(x), abs(s))), "silu(x) - silu(-x) = x"


def check_special_values(lib):
    """IEEE special values through the epilogues, the sum and the rounding:
    closed forms of binary64 arithmetic (inf * 0 and inf - inf are NaN, an
    infinite term dominates every finite one) and of the readings (ReLU is
    where(x > 0, x, 0), so NaN and -inf give +0; SiLU is x / (1 + exp(-x)),
    so +inf gives +inf and -inf gives -inf / inf = NaN)."""
    inf, nan = math.inf, math.nan
    ep = lambda x, e: oracle.epilogue64(x, e, lib)  # noqa: E731
    for e in EPIS:
        assert math.isnan(ep(nan, e)) == (e != "relu"), f"{e}(NaN)"
    for x, want in ((nan, 0.0), (inf, inf), (-inf, 0.0)):
        v = ep(x, "relu")
        assert v == want and math.copysign(1.0, v) == 1.0, f"relu({x}) = {v}"
    assert ep(inf, "silu") == inf and math.isnan(ep(-inf, "silu"))
    assert ep(inf, "identity") == inf and ep(-inf, "identity") == -inf
    for dtype in DTYPES:
        # rows of A: +inf at k=1; +inf at k=1 and -inf at k=2; NaN at k=3; ones
        # rows of B: ones; ones with 0 at k=1; minus ones
        Av = np.ones((1, 4, 5))
        Av[0, 0, 1] = inf
        Av[0, 1, 1], Av[0, 1, 2] = inf, -inf
        Av[0, 2, 3] = nan
        Bv = np.ones((1, 3, 5))
        Bv[0, 1, 1] = 0.0
        Bv[0, 2, :] = -1.0
        to_bits = {"f32": lambda v: v.astype(np.float32),
                   "f16": lambda v: v.astype(np.float16).view(np.uint16),
                   "bf16": lambda v: (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)}[dtype]
        C = oracle.gemm64(to_bits(Av), to_bits(Bv), dtype, "identity", lib=lib)
        want = np.array([[inf, nan, -inf], [nan, nan, nan], [nan, nan, nan], [5.0, 4.0, -5.0]])
        assert np.array_equal(np.isnan(C[0]), np.isnan(want)), f"{dtype}: NaN pattern {C[0]}"
        fin = ~np.isnan(want)
        assert np.array_equal(C[0][fin], want[fin]), f"{dtype}: {C[0]}"
        R = oracle.gemm64(to_bits(Av), to_bits(Bv), dtype, "relu", lib=lib)[0]
        assert np.array_equal(R, np.where(want > 0, want, 0.0)) and not np.any(np.signbit(R)), f"{dtype}: relu {R}"
        # rounding keeps infinities and NaN; the largest finite value times 2 overflows
        big = {"f32": float(np.finfo(np.float32).max), "f16": 65504.0, "bf16": float(np.array([0x7F7F0000], np.uint32).view(np.float32)[0])}[dtype]
        bits = oracle.round_to_dtype(np.array([inf, -inf, nan, 2 * big, -2 * big]), dtype, lib)
        back = _exact_values(bits, dtype)
        assert back[0] == inf and back[1] == -inf and math.isnan(back[2]), f"{dtype}: {back}"
        assert back[3] == inf and back[4] == -inf, f"{dtype}: overflow {back}"
        # RMSNorm: a row with an infinity has an infinite sum of squares, so
        # its scale 1/sqrt(inf) is 0: inf * 0 is NaN, finite elements become
        # signed zeros; a NaN anywhere in a row makes the whole row NaN
        x = to_bits(np.array([[inf, 1.0, -2.0], [1.0, nan, 1.0], [-inf, -inf, 3.0]]))
        y = oracle.rms_norm64(x, to_bits(np.ones(3)), 1e-6, dtype, lib=lib)
        assert math.isnan(y[0, 0]) and y[0, 1] == 0.0 and not np.signbit(y[0, 1]), f"{dtype}: {y[0]}"
        assert y[0, 2] == 0.0 and np.signbit(y[0, 2]), f"{dtype}: -2 * 0 is -0 ({y[0]})"
        assert np.isnan(y[1]).all() and np.isnan(y[2, :2]).all() and y[2, 2] == 0.0, f"{dtype}: {y[1:]}"


# ------------------------------------------------------------------ GEMM pins

def check_closed_form_identity_B(lib):
    rng = np.random.default_rng(10)
    for dtype in DTYPES:
        for epi in EPIS:
            L, M, K = 2, 9, 13
            A = _random_bits(rng, dtype, (L, M, K))
            if dtype == "f32":
                one, zero = np.float32(1.0), np.float32(0.0)
                B = np.zeros((L, K, K), np.float32)
            else:
                one = np.float16(1.0).view(np.uint16) if dtype == "f16" else np.uint16(0x3F80)
                zero = np.uint16(0)
                B = np.full((L, K, K), zero, np.uint16)
            for l in range(L):
                np.fill_diagonal(B[l], one)
            C = oracle.gemm64(A, B, dtype, epi, lib=lib)
            Av = _exact_values(A, dtype)
            want = np.vectorize(lambda v: oracle.epilogue64(v, epi, lib))(Av)
            assert np.array_equal(C, want), f"identity B: C != epi(A) ({dtype}, {epi})"
            if epi != "silu":
                bits = oracle.round_to_dtype(C, dtype, lib)
                if epi == "identity":
                    assert np.array_equal(bits.view(np.uint8), A.view(np.uint8)), "identity B: bits"


def check_closed_form_all_ones(lib):
    for dtype in DTYPES:
        for K in (1, 7, 128, 2048):
            if dtype == "f32":
                A = np.ones((1, 3, K), np.float32)
                B = np.ones((1, 5, K), np.float32)
            else:
                one = np.float16(1.0).view(np.uint16) if dtype == "f16" else np.uint16(0x3F80)
                A = np.full((1, 3, K), one, np.uint16)
                B = np.full((1, 5, K), one, np.uint16)
            for epi in ("identity", "relu"):
                C = oracle.gemm64(A, B, dtype, epi, lib=lib)
                assert np.all(C == float(K)), f"all-ones gives K ({dtype}, K={K})"
                bits = oracle.round_to_dtype(C, dtype, lib)
                assert np.all(oracle.widen(bits, dtype, lib) == float(K)), "K is exact in every dtype"
            C = oracle.gemm64(A, B, dtype, "silu", lib=lib)
            assert np.allclose(C, K / (1 + math.exp(-K)), rtol=1e-15, atol=0)


def check_bruteforce_fraction(lib):
    rng = np.random.default_rng(11)
    shapes = [(1, 1, 1, 1), (1, 2, 3, 4), (2, 3, 5, 7), (3, 7, 4, 6), (2, 6, 7, 5), (1, 5, 2, 7)]
    for dtype in DTYPES:
        for (L, M, N, K) in shapes:
            A = _random_bits(rng, dtype, (L, M, K))
            B = _random_bits(rng, dtype, (L, N, K))
            exact, mag = _frac_gemm(_exact_values(A, dtype), _exact_values(B, dtype))
            got = {e: oracle.gemm64(A, B, dtype, e, lib=lib) for e in EPIS}
            for l in range(L):
                for m in range(M):
                    for n in range(N):
                        s = exact[l][m][n]
                        bound = K * 2.0 ** -53 * float(mag[l][m][n])
                        gi = got["identity"][l, m, n]
                        assert abs(Fraction(gi) - s) <= Fraction(bound), \
                            f"sum off by more than K*u*sum|ab| ({dtype}, {(L, M, N, K)}, {(l, m, n)})"
                        gr = got["relu"][l, m, n]
                        assert gr == max(gi, 0.0) and not (gr == 0 and math.copysign(1, gr) < 0)
                        assert Fraction(gr) == _relu_exact(Fraction(gi))
                        ref = _silu_mp(s)
                        gs = got["silu"][l, m, n]
                        assert abs(gs - ref) <= 1e-13 * max(abs(ref), 1e-300) + bound * 1.2, \
                            f"silu of the sum ({dtype}, {(l, m, n)})"


def check_matmul_crosscheck(lib):
    rng = np.random.default_rng(12)
    for dtype in DTYPES:
        L, M, N, K = 2, 33, 70, 257
        A = _random_bits(rng, dtype, (L, M, K))
        B = _random_bits(rng, dtype, (L, N, K))
        Av, Bv = _exact_values(A, dtype), _exact_values(B, dtype)
        ref = np.matmul(Av, np.transpose(Bv, (0, 2, 1)))
        mag = np.matmul(np.abs(Av), np.transpose(np.abs(Bv), (0, 2, 1)))
        got = oracle.gemm64(A, B, dtype, "identity", lib=lib)
        assert np.all(np.abs(got - ref) <= 2 * K * 2.0 ** -53 * mag), f"numpy matmul cross-check ({dtype})"
        relu = oracle.gemm64(A, B, dtype, "relu", lib=lib)
        assert np.array_equal(relu, np.where(got > 0, got, 0.0))


def check_batch_and_entries(lib):
    rng = np.random.default_rng(13)
    for dtype in DTYPES:
        L, M, N, K = 3, 6, 11, 19
        A = _random_bits(rng, dtype, (L, M, K))
        B = _random_bits(rng, dtype, (L, N, K))
        full = oracle.gemm64(A, B, dtype, "silu", lib=lib)
        for l in range(L):
            one = oracle.gemm64(A[l:l + 1], B[l:l + 1], dtype, "silu", lib=lib)
            assert np.array_equal(one[0], full[l]), "batch independence"
        li = rng.integers(0, L, 50)
        mi = rng.integers(0, M, 50)
        ni = rng.integers(0, N, 50)
        ent = oracle.gemm_entries64(A, B, dtype, "silu", li, mi, ni, lib=lib)
        assert np.array_equal(ent, full[li, mi, ni]), "entries agree with the full GEMM"


def check_empty_K(lib):
    for dtype in DTYPES:
        st = np.float32 if dtype == "f32" else np.uint16
        A = np.zeros((2, 3, 0), st)
        B = np.zeros((2, 4, 0), st)
        for epi in EPIS:
            C = oracle.gemm64(A, B, dtype, epi, lib=lib)
            assert C.shape == (2, 3, 4) and np.all(C == 0.0), "K = 0 gives epilogue(0) = 0"


def check_grouped_vs_numpy(lib):
    """Grouped GEMM: every group's rows equal numpy's binary64 product of that
    group's rows with its own B (within the summation error bound); integer
    inputs exactly equal numpy's int64 product; rows in no group stay unwritten;
    empty groups and a group of one row are covered."""
    rng = np.random.default_rng(21)
    for dtype in DTYPES:
        G, N, K = 5, 37, 129
        sizes = [3, 0, 70, 1, 0]
        ends = np.cumsum(sizes).astype(np.int32)
        total_m = int(ends[-1]) + 4                       # 4 trailing rows in no group
        A = _random_bits(rng, dtype, (total_m, K))
        B = _random_bits(rng, dtype, (G, N, K))
        Av, Bv = _exact_values(A, dtype), _exact_values(B, dtype)
        got = oracle.gemm_grouped64(A, B, ends, dtype, "identity", lib=lib)
        relu = oracle.gemm_grouped64(A, B, ends, dtype, "relu", lib=lib)
        start = 0
        for g in range(G):
            end = int(ends[g])
            ref = Av[start:end] @ Bv[g].T
            mag = np.abs(Av[start:end]) @ np.abs(Bv[g]).T
            assert np.all(np.abs(got[start:end] - ref) <= 2 * K * 2.0 ** -53 * mag), f"group {g} ({dtype})"
            assert np.array_equal(relu[start:end], np.maximum(got[start:end], 0.0) + 0.0)
            start = end
        assert np.all(np.isnan(got[start:])), "rows in no group must stay unwritten"
        # integers: exact against numpy's int64 arithmetic, group by group
        Ai = rng.integers(-2, 3, (total_m, K))
        Bi = rng.integers(-2, 3, (G, N, K))
        to_bits = {"f32": lambda x: x.astype(np.float32),
                   "f16": lambda x: x.astype(np.float16).view(np.uint16),
                   "bf16": lambda x: (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)}[dtype]
        exact = oracle.gemm_grouped64(to_bits(Ai), to_bits(Bi), ends, dtype, "identity", lib=lib)
        start = 0
        for g in range(G):
            end = int(ends[g])
            assert np.array_equal(exact[start:end], (Ai[start:end] @ Bi[g].T).astype(np.float64)), f"int {g}"
            start = end
    # a single group covering every row is the dense GEMM of one batch
    A = _random_bits(rng, "bf16", (9, 40))
    B = _random_bits(rng, "bf16", (1, 6, 40))
    one = oracle.gemm_grouped64(A, B, np.array([9], np.int32), "bf16", "silu", lib=lib)
    dense = oracle.gemm64(A[None], B, "bf16", "silu", lib=lib)[0]
    assert np.array_equal(one, dense)


# ------------------------------------------------------------------ RMSNorm

def _rms_mp(xv, wv, eps):
    """RMSNorm of one row at 200 bits: x_j * w_j / sqrt(mean(x^2) + eps)."""
    import mpmath

    mpmath.mp.prec = 200
    xs = [mpmath.mpf(float(v)) for v in xv]
    ms = mpmath.fsum(v * v for v in xs) / len(xs)
    inv = 1 / mpmath.sqrt(ms + mpmath.mpf(float(eps)))
    return np.array([float(v * inv * mpmath.mpf(float(w))) for v, w in zip(xs, wv)])


def check_rms_norm_vs_torch_and_mp(lib):
    """RMSNorm agrees with torch.nn.functional.rms_norm run in binary64 on the
    exact input values (an implementation of its own) and, on short rows, with
    a 200-bit evaluation of the definition, for every dtype, ragged hidden
    sizes and random weights."""
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(31)
    for dtype in DTYPES:
        for rows, H, eps in [(5, 2048, 1e-6), (3, 37, 1e-5), (4, 1, 1e-6), (2, 3584, 0.0)]:
            x = _random_bits(rng, dtype, (rows, H), scale=3.0)
            w = _random_bits(rng, dtype, (H,))
            xv, wv = _exact_values(x, dtype), _exact_values(w, dtype)
            got = oracle.rms_norm64(x, w, eps, dtype, lib=lib)
            ref = F.rms_norm(torch.from_numpy(xv), (H,), weight=torch.from_numpy(wv), eps=eps).numpy()
            scale = np.abs(xv * wv) / np.sqrt((xv * xv).mean(axis=1, keepdims=True) + eps)
            assert np.all(np.abs(got - ref) <= 1e-12 * scale + 1e-300), f"vs torch ({dtype}, H={H})"
            if H <= 64:
                for r in range(rows):
                    mp = _rms_mp(xv[r], wv, eps)
                    assert np.all(np.abs(got[r] - mp) <= 4 * 2.0 ** -52 * scale[r] + 1e-300), f"vs mp ({dtype})"


def check_rms_norm_closed_forms(lib):
    """Closed forms: a constant row c with unit weight gives c / sqrt(c^2 + eps);
    with eps = 0 and c a power of two it gives exactly +-1; a zero row gives 0
    (eps keeps the reciprocal finite); a row much smaller than sqrt(eps) is
    scaled by about 1/sqrt(eps), since eps sits inside the square root."""
    def const(dtype, shape, v):     # v is exactly representable in every dtype used here
        if dtype == "f32":
            return np.full(shape, v, np.float32)
        if dtype == "f16":
            return np.full(shape, v, np.float16).view(np.uint16)
        return (np.full(shape, v, np.float32).view(np.uint32) >> 16).astype(np.uint16)

    for dtype in DTYPES:
        H = 64
        w = const(dtype, (H,), 1.0)
        for c, eps in [(2.0, 0.0), (-0.5, 0.0), (0.75, 1e-6), (3.0, 0.25)]:
            x = const(dtype, (1, H), c)
            got = oracle.rms_norm64(x, w, eps, dtype, lib=lib)
            want = c / math.sqrt(c * c + eps)
            assert np.all(np.abs(got - want) <= 2 * 2.0 ** -52 * abs(want)), f"constant row {c} ({dtype})"
            if eps == 0.0:
                assert np.all(got == math.copysign(1.0, c)), "power-of-two row must normalise exactly"
        zero = np.zeros((2, H), np.float32 if dtype == "f32" else np.uint16)
        got = oracle.rms_norm64(zero, w, 1e-6, dtype, lib=lib)
        assert np.all(got == 0.0), "zero row"
    # tiny row in fp32: x = 2^-20 everywhere, eps = 1e-6  ->  y = x / sqrt(x^2 + eps)
    H = 16
    x = np.full((1, H), 2.0 ** -20, np.float32)
    got = oracle.rms_norm64(x, np.ones(H, np.float32), 1e-6, "f32", lib=lib)
    want = 2.0 ** -20 / math.sqrt(2.0 ** -40 + 1e-6)
    assert abs(got[0, 0] - want) <= 4 * 2.0 ** -52 * want, "eps belongs inside the square root"


def check_rms_norm_invariants(lib):
    """Rows are independent (permuting rows permutes the result bitwise); with
    eps = 0 scaling a row by a power of two leaves it unchanged bitwise and the
    normalised row (unit weight) has mean square 1; the weight scales each
    column (result with weight w == result with unit weight times w)."""
    rng = np.random.default_rng(32)
    rows, H = 6, 300
    x = rng.standard_normal((rows, H)).astype(np.float32)
    w = rng.standard_normal(H).astype(np.float32)
    ones = np.ones(H, np.float32)
    base = oracle.rms_norm64(x, w, 1e-6, "f32", lib=lib)
    perm = rng.permutation(rows)
    assert np.array_equal(oracle.rms_norm64(x[perm], w, 1e-6, "f32", lib=lib), base[perm]), "rows"
    n0 = oracle.rms_norm64(x, ones, 0.0, "f32", lib=lib)
    assert np.array_equal(oracle.rms_norm64(x * np.float32(8.0), ones, 0.0, "f32", lib=lib), n0), "scale"
    assert np.all(np.abs((n0 * n0).mean(axis=1) - 1.0) <= 1e-13), "mean square of a normalised row"
    unit = oracle.rms_norm64(x, ones, 1e-6, "f32", lib=lib)
    assert np.array_equal(unit * w.astype(np.float64), base), "weight per column"


ALL_CHECKS = [
    check_widen_f16_exhaustive,
    check_widen_bf16_exhaustive,
    check_round_bf16_midpoints,
    check_round_f16_vs_numpy,
    check_round_f32_vs_cast,
    check_epilogue_values,
    check_special_values,
    check_closed_form_identity_B,
    check_closed_form_all_ones,
    check_bruteforce_fraction,
    check_matmul_crosscheck,
    check_batch_and_entries,
    check_empty_K,
    check_grouped_vs_numpy,
    check_rms_norm_vs_torch_and_mp,
    check_rms_norm_closed_forms,
    check_rms_norm_invariants,
]
