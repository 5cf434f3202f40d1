"""Full-size parity of the three large workloads, in the launch configuration
the benchmark times (the automatic plan) and, for the K-heavy batched shape,
through the split-K path as well (2 and 4 splits: fp32 partial sums added in
ascending split order, then the epilogue once).

What each test covers (the whole output unless it says otherwise):
  - bf16 512x5632x2048 ReLU: every output against the oracle, random inputs
    within the tolerance, integer inputs bit for bit.
  - fp16 8192^3 identity: integer inputs, every output bit for bit, through
    per-block digests of the oracle's result (tests/golden/full_int_digests.txt,
    written by tests/golden/make_full_digests.py, which calls only the oracle);
    random inputs on 64 whole rows and 64 whole columns, one in every 128-row
    and every 128-column block (so every output tile is crossed), against
    the oracle.
  - bf16 L=8 512x3584x18944 SiLU, at S = auto, 2 and 4: integer inputs (ReLU:
    SiLU is never bit-exact) every output bit for bit through the digests;
    random inputs on one whole batch and, in every batch, 8 whole rows and 28
    whole columns crossing every tile, against the oracle.

Run on an MI355X:  python -u -m pytest tests -m gpu -x -v --timeout 300 --timeout-method thread
"""
from __future__ import annotations

import functools
import hashlib
import os

import numpy as np
import pytest

import tiled_dense_gemm_mkl_amd as gm
from tiled_dense_gemm_mkl_amd import workloads
from gpu_helpers import TOL, assert_bits_equal, assert_close, require_gpu, run_gemm, to_device, widen_bits

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
DIGESTS = os.path.join(HERE, "golden", "full_int_digests.txt")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@functools.lru_cache(maxsize=4)
def _inputs(key: str, integer: bool):
    return workloads.make_inputs(workloads.WORKLOADS[key], integer=integer)


def _digests(key: str, epi: str):
    """{(batch, first row): (rows, digest)} of the stored oracle digests."""
    out = {}
    with open(DIGESTS) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, e, l, m0, rows, h = line.split()
            if k == key and e == epi:
                out[(int(l), int(m0))] = (int(rows), h)
    assert out, f"no digests stored for {key} {epi}"
    return out


def _check_digests(C: np.ndarray, key: str, epi: str, what: str):
    """Hash every block of rows of C (stored bits) as the digest script does
    and compare with the stored digests of the oracle's result."""
    want = _digests(key, epi)
    L, M, _ = C.shape
    bad = []
    seen = 0
    for (l, m0), (rows, h) in sorted(want.items()):
        blk = C[l, m0:m0 + rows]
        assert blk.shape[0] == rows
        got = hashlib.sha256(blk.astype(blk.dtype.newbyteorder("<"), copy=False).tobytes()).hexdigest()[:32]
        seen += rows
        if got != h:
            bad.append((l, m0))
    assert seen == L * M, f"{what}: digests cover {seen} of {L * M} rows"
    assert not bad, f"{what}: {len(bad)} of {len(want)} row blocks differ from the oracle, first {bad[:4]}"


# ---------------------------------------------------------------- bf16 512x5632x2048 ReLU (headline)

HEADLINE = "bf16_512x5632x2048_relu"


def test_headline_every_output_random_inputs(orc):
    w = workloads.WORKLOADS[HEADLINE]
    A, B = _inputs(HEADLINE, False)
    C = run_gemm(A, B, w.dtype, w.epilogue)
    ref = orc.gemm64(A, B, w.dtype, w.epilogue)
    err = assert_close(C, ref, A, B, w.dtype, w.K, HEADLINE)
    print(f"{HEADLINE}: every output, err {err:.3e} (tol {TOL[w.dtype]:.0e})")


def test_headline_every_output_integer_inputs_bit_exact(orc):
    w = workloads.WORKLOADS[HEADLINE]
    A, B = _inputs(HEADLINE, True)
    C = run_gemm(A, B, w.dtype, w.epilogue)
    ref = orc.round_to_dtype(orc.gemm64(A, B, w.dtype, w.epilogue), w.dtype)
    assert_bits_equal(C, ref, f"{HEADLINE} integer")


# ---------------------------------------------------------------- fp16 8192^3 identity

SQUARE = "f16_8192x8192x8192_identity"


def test_square_every_output_integer_inputs_bit_exact():
    w = workloads.WORKLOADS[SQUARE]
    A, B = _inputs(SQUARE, True)
    C = run_gemm(A, B, w.dtype, w.epilogue)
    _check_digests(C, SQUARE, w.epilogue, f"{SQUARE} integer")


def _crossing(n: int, block: int, seed: int) -> np.ndarray:
    """One index in every block of `block` (a different offset in each)."""
    rng = np.random.default_rng(seed)
    idx = [b + int(rng.integers(0, min(block, n - b))) for b in range(0, n, block)]
    return np.array(sorted(set(idx + [0, n - 1])))


def test_square_random_inputs_rows_and_columns_crossing_every_tile(orc):
    w = workloads.WORKLOADS[SQUARE]
    A, B = _inputs(SQUARE, False)
    C = run_gemm(A, B, w.dtype, w.epilogue)
    rows = _crossing(w.M, 128, 41)
    cols = _crossing(w.N, 128, 42)
    ref_rows = orc.gemm64(np.ascontiguousarray(A[:, rows, :]), B, w.dtype, w.epilogue)
    err_r = assert_close(C[:, rows, :], ref_rows, A, B, w.dtype, w.K, f"{SQUARE} rows")
    ref_cols = orc.gemm64(A, np.ascontiguousarray(B[:, cols, :]), w.dtype, w.epilogue)
    err_c = assert_close(C[:, :, cols], ref_cols, A, B, w.dtype, w.K, f"{SQUARE} columns")
    assert np.all(np.isfinite(widen_bits(C, w.dtype)))
    print(f"{SQUARE}: {rows.size} whole rows err {err_r:.3e}, {cols.size} whole columns err {err_c:.3e}")


# ---------------------------------------------------------------- bf16 L=8 512x3584x18944 SiLU, split-K path

KHEAVY = "bf16_L8_512x3584x18944_silu"
SPLITS = (None, 2, 4)   # None: the automatic plan (the benchmark's launch configuration)


def _run_splits(A, B, dtype, epi):
    """{split: C} for every split of SPLITS, operands uploaded once."""
    import torch

    a, b = to_device(A, dtype), to_device(B, dtype)
    out = {}
    for S in SPLITS:
        kw = {} if S is None else {"split_k": S}
        if S is not None:
            plan = gm.get_plan(a.shape[1], b.shape[1], a.shape[2], a.shape[0], gm.DTYPE_CODES[dtype],
                               gm.EPILOGUE_CODES[epi], gm.make_opts(split_k=S))
            assert plan["split_k"] == S and plan["workspace_bytes"] > 0 and plan["streamk"] == 0
        c = gm.gemm(a, b, epi, **kw)
        torch.cuda.synchronize()
        out[S] = workloads.torch_to_storage(c)
        del c
    del a, b
    torch.cuda.empty_cache()
    return out


def test_k_heavy_every_output_integer_inputs_bit_exact_through_splits():
    w = workloads.WORKLOADS[KHEAVY]
    A, B = _inputs(KHEAVY, True)
    for S, C in _run_splits(A, B, w.dtype, "relu").items():
        _check_digests(C, KHEAVY, "relu", f"{KHEAVY} integer relu S={S or 'auto'}")


def test_k_heavy_random_inputs_through_splits(orc):
    w = workloads.WORKLOADS[KHEAVY]
    A, B = _inputs(KHEAVY, False)
    outs = _run_splits(A, B, w.dtype, w.epilogue)
    l_full = 3
    ref_batch = orc.gemm64(A[l_full:l_full + 1], B[l_full:l_full + 1], w.dtype, w.epilogue)
    rows = _crossing(w.M, 64, 51)
    cols = _crossing(w.N, 128, 52)
    ref_rows = orc.gemm64(np.ascontiguousarray(A[:, rows, :]), B, w.dtype, w.epilogue)
    ref_cols = orc.gemm64(A, np.ascontiguousarray(B[:, cols, :]), w.dtype, w.epilogue)
    for S, C in outs.items():
        tag = f"{KHEAVY} S={S or 'auto'}"
        e1 = assert_close(C[l_full:l_full + 1], ref_batch, A, B, w.dtype, w.K, f"{tag} batch {l_full}")
        e2 = assert_close(C[:, rows, :], ref_rows, A, B, w.dtype, w.K, f"{tag} rows")
        e3 = assert_close(C[:, :, cols], ref_cols, A, B, w.dtype, w.K, f"{tag} columns")
        assert np.all(np.isfinite(widen_bits(C, w.dtype)))
        print(f"{tag}: batch {l_full} err {e1:.3e}, {rows.size} rows x 8 err {e2:.3e}, "
              f"{cols.size} columns x 8 err {e3:.3e}")
    # each split's result is reproducible from run to run
    again = _run_splits(A, B, w.dtype, w.epilogue)
    for S in SPLITS:
        assert_bits_equal(again[S], outs[S], f"{KHEAVY} S={S or 'auto'} run-to-run")
