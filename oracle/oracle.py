"""ctypes front end of the C oracle (gemm_oracle.c).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Inputs are numpy arrays holding the *stored bits* of the operands:
``float32`` arrays for fp32, ``uint16`` arrays for fp16 and bf16.  Shapes are
A ``[L, M, K]``, B ``[L, N, K]`` (K contiguous); results are ``[L, M, N]``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_oracle.c")
_LIB = os.path.join(_HERE, "libgemm_oracle.so")

DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
EPILOGUES = {"identity": 0, "relu": 1, "silu": 2}

_lib = None


def compile_source(src: str, out: str) -> str:
    """gcc -O2 with OpenMP, no FP contraction and no fast-math, as a shared object."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-std=c11", "-shared", "-fPIC", src, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile gemm_oracle.c into libgemm_oracle.so beside it."""
    if force or not os.path.exists(_LIB):
        compile_source(_SRC, _LIB)
    return _LIB


def load(path: str | None = None):
    """Load the oracle library (the default build, or another build at path)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_gemm.argtypes = [vp, vp, vp, i64, i64, i64, i64,
                                ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.oracle_gemm.restype = ctypes.c_int
    lib.oracle_gemm_entries.argtypes = [vp, vp, i64, i64, i64, i64,
                                        ctypes.c_int, ctypes.c_int,
                                        vp, vp, vp, i64, vp, ctypes.c_int]
    lib.oracle_gemm_entries.restype = ctypes.c_int
    lib.oracle_gemm_grouped.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int]
    lib.oracle_gemm_grouped.restype = ctypes.c_int
    lib.oracle_rms_norm.argtypes = [vp, vp, vp, i64, i64, ctypes.c_double, ctypes.c_int, ctypes.c_int]
    lib.oracle_rms_norm.restype = ctypes.c_int
    lib.oracle_round.argtypes = [vp, vp, i64, ctypes.c_int]
    lib.oracle_round.restype = None
    lib.oracle_widen.argtypes = [vp, vp, i64, ctypes.c_int]
    lib.oracle_widen.restype = None
    lib.oracle_epilogue.argtypes = [ctypes.c_double, ctypes.c_int]
    lib.oracle_epilogue.restype = ctypes.c_double
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = ctypes.c_int
    return lib


def _storage(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def _check(x: np.ndarray, dtype: str) -> np.ndarray:
    want = _storage(dtype)
    if x.dtype != want:
        raise TypeError(f"oracle expects {np.dtype(want).name} storage for {dtype}, got {x.dtype}")
    return np.ascontiguousarray(x)


def _ptr(x: np.ndarray):
    return x.ctypes.data_as(ctypes.c_void_p)


def gemm64(A: np.ndarray, B: np.ndarray, dtype: str, epilogue: str,
           nthreads: int = 0, lib=None) -> np.ndarray:
    """epilogue(sum_k A[l,m,k] B[l,n,k]) in binary64, shape [L, M, N]."""
    A = _check(A, dtype)
    B = _check(B, dtype)
    L, M, K = A.shape
    Lb, N, Kb = B.shape
    if (Lb, Kb) != (L, K):
        raise ValueError(f"shape mismatch A{A.shape} B{B.shape}")
    C = np.empty((L, M, N), dtype=np.float64)
    (lib or load()).oracle_gemm(_ptr(A), _ptr(B), _ptr(C), M, N, K, L,
                                DTYPES[dtype], EPILOGUES[epilogue], nthreads)
    return C


def gemm_entries64(A: np.ndarray, B: np.ndarray, dtype: str, epilogue: str,
                   l_idx, m_idx, n_idx, nthreads: int = 0, lib=None) -> np.ndarray:
    """Selected entries C64[l_i, m_i, n_i] of gemm64, computed one by one."""
    A = _check(A, dtype)
    B = _check(B, dtype)
    L, M, K = A.shape
    N = B.shape[1]
    li = np.ascontiguousarray(l_idx, dtype=np.int64)
    mi = np.ascontiguousarray(m_idx, dtype=np.int64)
    ni = np.ascontiguousarray(n_idx, dtype=np.int64)
    if not (li.shape == mi.shape == ni.shape):
        raise ValueError("index arrays must have one shape")
    if li.size and (li.min() < 0 or li.max() >= L or mi.min() < 0 or mi.max() >= M
                    or ni.min() < 0 or ni.max() >= N):
        raise IndexError("entry index out of range")
    out = np.empty(li.shape, dtype=np.float64)
    (lib or load()).oracle_gemm_entries(_ptr(A), _ptr(B), M, N, K, L, DTYPES[dtype],
                                        EPILOGUES[epilogue], _ptr(li), _ptr(mi), _ptr(ni),
                                        li.size, _ptr(out), nthreads)
    return out


def gemm_grouped64(A: np.ndarray, B: np.ndarray, offs: np.ndarray, dtype: str, epilogue: str,
                   nthreads: int = 0, lib=None) -> np.ndarray:
    """Grouped GEMM in binary64: A [total_m, K], B [G, N, K] (stored bits), offs
    int32 [G] cumulative row ends.  Rows in no group come back as NaN."""
    lib = lib or load()
    A = _check(A, dtype)
    B = _check(B, dtype)
    offs = np.ascontiguousarray(offs, dtype=np.int32)
    total_m, K = A.shape
    G, N, Kb = B.shape
    assert Kb == K and offs.shape == (G,)
    C = np.full((total_m, N), np.nan)
    st = lib.oracle_gemm_grouped(_ptr(A), _ptr(B), _ptr(C), _ptr(offs), G, total_m, N, K,
                                 DTYPES[dtype], EPILOGUES[epilogue], nthreads)
    if st < 0:
        raise ValueError("group offsets must be non-decreasing within [0, total_m]")
    return C


def rms_norm64(x: np.ndarray, w: np.ndarray, eps: float, dtype: str,
               nthreads: int = 0, lib=None) -> np.ndarray:
    """RMSNorm of the rows of x ([rows, H], stored bits) with weight w ([H]) in
    binary64, unrounded.  eps is used as given."""
    x = _check(x, dtype)
    w = _check(w, dtype)
    rows, H = x.shape
    if w.shape != (H,):
        raise ValueError(f"weight shape {w.shape} does not match hidden size {H}")
    y = np.empty((rows, H), dtype=np.float64)
    (lib or load()).oracle_rms_norm(_ptr(x), _ptr(w), _ptr(y), rows, H, float(eps),
                                    DTYPES[dtype], nthreads)
    return y


def round_to_dtype(y64: np.ndarray, dtype: str, lib=None) -> np.ndarray:
    """Round binary64 values once to dtype; returns the stored bits."""
    y = np.ascontiguousarray(y64, dtype=np.float64)
    out = np.empty(y.shape, dtype=_storage(dtype))
    (lib or load()).oracle_round(_ptr(y), _ptr(out), y.size, DTYPES[dtype])
    return out


def widen(x: np.ndarray, dtype: str, lib=None) -> np.ndarray:
    """Stored bits of dtype -> exact binary64 values."""
    x = _check(x, dtype)
    out = np.empty(x.shape, dtype=np.float64)
    (lib or load()).oracle_widen(_ptr(x), _ptr(out), x.size, DTYPES[dtype])
    return out


def threads(lib=None) -> int:
    """OpenMP threads the oracle uses on this host."""
    return int((lib or load()).oracle_threads())


def epilogue64(x: float, epilogue: str, lib=None) -> float:
    return (lib or load()).oracle_epilogue(float(x), EPILOGUES[epilogue])


def gemm_rounded(A: np.ndarray, B: np.ndarray, dtype: str, epilogue: str,
                 nthreads: int = 0, lib=None):
    """(binary64 result, result rounded once to dtype as stored bits)."""
    y = gemm64(A, B, dtype, epilogue, nthreads, lib)
    return y, round_to_dtype(y, dtype, lib)
