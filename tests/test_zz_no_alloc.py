"""GPU tests of gemm_mkl_noalloc, the entry point that allocates nothing: its
split-K partial sums and repacked operands live in the library's fixed device
scratch.  Its results are compared, through the C ABI, with gemm_mkl_ex's on
the same plan (bit for bit: the same kernels in the same order) and with the
oracle (integer inputs bit-exact, random inputs within the tolerance), on two
calls in a row, the second one smaller (the scratch keeps the first call's
contents)."""
from __future__ import annotations

import numpy as np
import pytest

import tiled_dense_gemm_mkl_amd as gm
from tiled_dense_gemm_mkl_amd import workloads
from gpu_helpers import assert_bits_equal, assert_close, require_gpu, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _call(entry, a, b, c, M, N, K, L, dtype, epi, opts):
    import torch

    st = entry(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, L, gm.DTYPE_CODES[dtype],
               gm.EPILOGUE_CODES[epi], torch.cuda.current_stream().cuda_stream, opts)
    assert st == 0, gm.status_string(st)


def _both(A, B, dtype, epi, opts_kw):
    """(noalloc result, gemm_mkl_ex result) as stored bits, same options."""
    import torch

    L, M, K = A.shape
    N = B.shape[1]
    a, b = to_device(A, dtype), to_device(B, dtype)
    c1 = torch.full((L, M, N), 7.0, dtype=a.dtype, device=a.device)
    c2 = torch.full((L, M, N), -7.0, dtype=a.dtype, device=a.device)
    _call(gm.gemm_mkl_noalloc, a, b, c1, M, N, K, L, dtype, epi, gm.make_opts(**opts_kw))
    _call(gm.gemm_mkl_ex, a, b, c2, M, N, K, L, dtype, epi, gm.make_opts(**opts_kw))
    torch.cuda.synchronize()
    return workloads.torch_to_storage(c1), workloads.torch_to_storage(c2)


# (dtype, M, N, K, L, options): the first call of each pair is the larger one
PAIRS = [
    # split-K partials in the scratch: 4 * 512 * 1536 * 4 B = 12 MB, then 1.4 MB
    (("bf16", 512, 1536, 4096, 1, dict(split_k=4)), ("bf16", 200, 300, 1032, 2, dict(split_k=3))),
    # fp32 split plan of the 128 x 2048 x 2048 workload, then a smaller one
    (("f32", 128, 2048, 2048, 1, dict()), ("f32", 96, 520, 1000, 1, dict(split_k=2))),
    # repacked operands (K * element bytes not a multiple of 16) plus a split
    (("f16", 300, 700, 2047, 2, dict(split_k=2)), ("f16", 33, 17, 13, 1, dict())),
]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0][0]}-{p[0][1]}x{p[0][2]}x{p[0][3]}")
def test_noalloc_matches_gemm_mkl_ex_twice_in_a_row(orc, pair):
    for i, (dtype, M, N, K, L, kw) in enumerate(pair):
        Ai, Bi = workloads.random_operands(dtype, M, N, K, L, seed=900 + i, integer=True)
        c_na, c_ex = _both(Ai, Bi, dtype, "relu", kw)
        ref = orc.round_to_dtype(orc.gemm64(Ai, Bi, dtype, "relu"), dtype)
        assert_bits_equal(c_na, ref, f"noalloc integer {dtype} {M}x{N}x{K}x{L} {kw}")
        assert_bits_equal(c_ex, ref, f"ex integer {dtype} {M}x{N}x{K}x{L} {kw}")
        A, B = workloads.random_operands(dtype, M, N, K, L, seed=910 + i)
        c_na, c_ex = _both(A, B, dtype, "silu", kw)
        assert_bits_equal(c_na, c_ex, f"noalloc vs ex {dtype} {M}x{N}x{K}x{L} {kw}")
        assert_close(c_na, orc.gemm64(A, B, dtype, "silu"), A, B, dtype, K, f"noalloc {dtype} {kw}")


def test_noalloc_plan_beyond_the_scratch_is_rejected_and_C_untouched():
    import torch

    # a forced 16-way split of 512 x 4096 partials needs 128 MiB > 32 MiB
    M, N, K, L = 512, 4096, 2048, 1
    need = gm.get_plan(M, N, K, L, gm.BF16, gm.EPI_RELU, gm.make_opts(split_k=16))["workspace_bytes"]
    assert need > gm.NOALLOC_SCRATCH_BYTES
    A, B = workloads.random_operands("bf16", M, N, K, L, seed=5)
    a, b = to_device(A, "bf16"), to_device(B, "bf16")
    c = torch.full((L, M, N), 3.0, dtype=a.dtype, device=a.device)
    st = gm.gemm_mkl_noalloc(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, L, gm.BF16, gm.EPI_RELU,
                             torch.cuda.current_stream().cuda_stream, gm.make_opts(split_k=16))
    assert st == -4
    torch.cuda.synchronize()
    assert torch.all(c == 3.0).item()
    # the automatic plan of the same shape fits (it only takes splits that fit)
    st = gm.gemm_mkl_noalloc(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, L, gm.BF16, gm.EPI_RELU,
                             torch.cuda.current_stream().cuda_stream, None)
    assert st == 0
    ref = gm.gemm(a, b, "relu")
    torch.cuda.synchronize()
    C = workloads.torch_to_storage(c)
    assert np.isfinite(C.astype(np.float64)).all()
    plan = gm.get_plan(M, N, K, L, gm.BF16, gm.EPI_RELU)
    if plan["workspace_bytes"] <= gm.NOALLOC_SCRATCH_BYTES:
        assert_bits_equal(C, workloads.torch_to_storage(ref), "automatic plan, noalloc vs gemm")
