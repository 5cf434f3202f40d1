"""Helpers of the GPU parity tests: device round trips through the C ABI and
the tolerance metric.

    err = max |C_gpu - C_ref64| / (K * max|A| * max|B|)

must stay <= 1e-6 for fp32 and <= 1e-2 for fp16/bf16 on random inputs; with
integer-valued inputs every fp32 partial sum is exact, so the GPU result must
equal the oracle's single rounding bit for bit (identity and ReLU).
"""
from __future__ import annotations

import numpy as np
import pytest

import tiled_dense_gemm_mkl_amd as gm
from tiled_dense_gemm_mkl_amd import workloads

TOL = {"f32": 1e-6, "f16": 1e-2, "bf16": 1e-2}


def gpu_available() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


def require_gpu():
    if not gpu_available():
        pytest.skip("no GPU in this environment")
    gm.load()  # raises if the HIP library is missing: no silent fallback


def to_device(bits: np.ndarray, dtype: str):
    return workloads.storage_to_torch(np.ascontiguousarray(bits), dtype).cuda()


def run_gemm(A: np.ndarray, B: np.ndarray, dtype: str, epilogue: str, **kw) -> np.ndarray:
    """Upload, call gemm_mkl_ex through the binding, synchronise, download bits."""
    import torch

    a = to_device(A, dtype)
    b = to_device(B, dtype)
    c = gm.gemm(a, b, epilogue, **kw)
    torch.cuda.synchronize()
    return workloads.torch_to_storage(c)


def widen_bits(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Stored bits -> float64 (numpy/bit arithmetic only, no oracle code)."""
    if dtype == "f32":
        return bits.astype(np.float64)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def scale(A: np.ndarray, B: np.ndarray, dtype: str, K: int) -> float:
    ma = np.max(np.abs(widen_bits(A, dtype))) if A.size else 0.0
    mb = np.max(np.abs(widen_bits(B, dtype))) if B.size else 0.0
    return K * ma * mb


def tol_error(C_bits: np.ndarray, C64: np.ndarray, A, B, dtype: str, K: int) -> float:
    s = scale(A, B, dtype, K)
    diff = np.max(np.abs(widen_bits(C_bits, dtype) - C64)) if C64.size else 0.0
    if s == 0.0:
        return 0.0 if diff == 0.0 else float("inf")
    return float(diff / s)


def assert_close(C_bits, C64, A, B, dtype, K, what=""):
    assert np.all(np.isfinite(widen_bits(C_bits, dtype))), f"non-finite output {what}"
    err = tol_error(C_bits, C64, A, B, dtype, K)
    assert err <= TOL[dtype], f"{what}: err {err:.3e} > {TOL[dtype]:.0e}"
    return err


def _as_uint(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    return x.view({1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[x.itemsize])


def assert_bits_equal(C_bits, ref_bits, what=""):
    a, b = _as_uint(C_bits), _as_uint(ref_bits)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    if not np.array_equal(a, b):
        bad = np.nonzero(a.reshape(-1) != b.reshape(-1))[0]
        raise AssertionError(f"{what}: {bad.size} of {a.size} elements differ; first flat indices {bad[:5].tolist()}")


def sample_indices(L: int, M: int, N: int, count: int, seed: int):
    """Random entries plus the four corners and a ragged-edge band of every batch."""
    rng = np.random.default_rng(seed)
    li = list(rng.integers(0, L, count))
    mi = list(rng.integers(0, M, count))
    ni = list(rng.integers(0, N, count))
    for l in {0, L - 1}:
        for m in (0, 1, M // 2, M - 2, M - 1):
            for n in (0, 1, N // 2, N - 2, N - 1):
                if 0 <= m < M and 0 <= n < N:
                    li.append(l)
                    mi.append(m)
                    ni.append(n)
    return np.array(li), np.array(mi), np.array(ni)
