"""GPU checks of the repacked path: operands whose rows (K elements) or base
pointers are not 16-byte aligned are copied into zero-padded rows of Kp
elements in the workspace, and the tile kernels run at Kp.

  - The result equals, bit for bit, the same plan run on operands padded with
    zeros by the host (the aligned path at Kp): the zeros add nothing.
  - Integer inputs match the oracle bit for bit; random inputs meet the
    tolerance, on ragged shapes with batches and forced splits.
  - Only A, or only B, off a 16-byte boundary: that operand alone is repacked.
  - A caller workspace must also hold the repacked copies; a smaller one is
    refused before anything is launched (C untouched).
"""
import numpy as np
import pytest

import tiled_dense_gemm_mkl_amd as gm
from tiled_dense_gemm_mkl_amd import workloads
from gpu_helpers import TOL, assert_bits_equal, assert_close, require_gpu, run_gemm, to_device

pytestmark = pytest.mark.gpu

EB = {"f32": 4, "f16": 2, "bf16": 2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _pad(X, Kp):
    out = np.zeros(X.shape[:-1] + (Kp,), dtype=X.dtype)
    out[..., :X.shape[-1]] = X
    return out


def _round256(n):
    return (n + 255) // 256 * 256


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", [(512, 5632, 2047, 1), (300, 700, 1001, 2), (33, 17, 13, 3), (1000, 1100, 521, 1)],
                         ids=lambda s: "x".join(map(str, s)))
def test_repacked_equals_host_padded(orc, dtype, shape):
    M, N, K, L = shape
    vec = 16 // EB[dtype]
    Kp = (K + vec - 1) // vec * vec
    plan = gm.get_plan(M, N, K, L, gm.DTYPE_CODES[dtype], gm.EPI_RELU)
    assert plan["packed"] == 1
    fixed = dict(config_id=plan["config_id"], prefetch_stages=plan["prefetch_stages"], split_k=plan["split_k"])
    A, B = workloads.random_operands(dtype, M, N, K, L, seed=K, dist_a=("normal", 1.0), dist_b=("normal", 1.0))
    C = run_gemm(A, B, dtype, "relu", **fixed)
    Cpad = run_gemm(_pad(A, Kp), _pad(B, Kp), dtype, "relu", **fixed)
    assert_bits_equal(C, Cpad, f"{dtype} {shape}")
    Ai, Bi = workloads.random_operands(dtype, M, N, K, L, seed=K + 1, integer=True)
    Ci = run_gemm(Ai, Bi, dtype, "identity")
    li, mi, ni = np.meshgrid(np.arange(L), np.arange(min(M, 64)), np.arange(min(N, 64)), indexing="ij")
    ref = orc.round_to_dtype(orc.gemm_entries64(Ai, Bi, dtype, "identity", li.ravel(), mi.ravel(), ni.ravel()), dtype)
    assert_bits_equal(Ci[li.ravel(), mi.ravel(), ni.ravel()], ref, f"{dtype} {shape} integer")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("split", [2, 3])
def test_repacked_with_forced_split(orc, dtype, split):
    M, N, K, L = 200, 300, 1003, 2
    A, B = workloads.random_operands(dtype, M, N, K, L, seed=split)
    plan = gm.get_plan(M, N, K, L, gm.DTYPE_CODES[dtype], gm.EPI_SILU, gm.make_opts(split_k=split))
    assert plan["packed"] == 1 and plan["split_k"] == split
    C = run_gemm(A, B, dtype, "silu", split_k=split)
    assert_close(C, orc.gemm64(A, B, dtype, "silu"), A, B, dtype, K, f"{dtype} S={split}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("which", ["A", "B", "both"])
def test_one_operand_off_a_16_byte_boundary(orc, dtype, which):
    import torch

    M, N, K, L = 130, 90, 96, 2
    A, B = workloads.random_operands(dtype, M, N, K, L, seed=7)

    def shifted(X):       # the same values, starting one element past a 16-byte boundary
        big = to_device(np.concatenate([X.reshape(-1)[:1], X.reshape(-1)]), dtype)
        return big[1:].view(X.shape)

    a = shifted(A) if which in ("A", "both") else to_device(A, dtype)
    b = shifted(B) if which in ("B", "both") else to_device(B, dtype)
    assert (a.data_ptr() % 16 != 0) == (which in ("A", "both"))
    c = gm.gemm(a, b, "relu")
    torch.cuda.synchronize()
    ref = orc.gemm64(A, B, dtype, "relu")
    assert_close(workloads.torch_to_storage(c), ref, A, B, dtype, K, f"{dtype} {which} shifted")
    aligned = run_gemm(A, B, dtype, "relu")
    assert_bits_equal(workloads.torch_to_storage(c), aligned, f"{dtype} {which} shifted vs aligned")


def test_caller_workspace_must_hold_the_repacked_operands(orc):
    import torch

    dtype, M, N, K, L = "bf16", 64, 80, 13, 1
    Kp = 16
    A, B = workloads.random_operands(dtype, M, N, K, L, seed=3)
    a, b = to_device(A, dtype), to_device(B, dtype)
    need = _round256(L * M * Kp * 2) + _round256(L * N * Kp * 2)
    assert gm.get_plan(M, N, K, L, gm.BF16, gm.EPI_RELU)["workspace_bytes"] == need
    sentinel = -7.0
    for size, status in ((need - 256, -4), (need, 0)):
        ws = torch.empty(size, dtype=torch.uint8, device="cuda")
        c = torch.full((L, M, N), sentinel, dtype=torch.bfloat16, device="cuda")
        opts = gm.make_opts(workspace_ptr=ws.data_ptr(), workspace_bytes=size)
        st = gm.gemm_mkl_ex(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, L, gm.BF16, gm.EPI_RELU,
                            torch.cuda.current_stream().cuda_stream, opts)
        torch.cuda.synchronize()
        assert st == status
        if status != 0:
            assert bool((c == sentinel).all()), "C was written by a refused call"
        else:
            assert_close(workloads.torch_to_storage(c), orc.gemm64(A, B, dtype, "relu"), A, B, dtype, K,
                         "caller workspace")


# ------------------------------------------------------------------ grouped GEMM

def _grouped_run(A, B, offs, dtype, epilogue, shift_a=False):
    import torch

    a = to_device(A, dtype)
    if shift_a:   # the same values one element past a 16-byte boundary
        big = to_device(np.concatenate([A.reshape(-1)[:1], A.reshape(-1)]), dtype)
        a = big[1:].view(A.shape)
    b = to_device(B, dtype)
    o = torch.from_numpy(np.ascontiguousarray(offs, dtype=np.int32)).cuda()
    c = gm.gemm_grouped(a, b, o, epilogue)
    torch.cuda.synchronize()
    return workloads.torch_to_storage(c)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("K,shift_a", [(1001, False), (13, False), (96, True)], ids=["K1001", "K13", "shiftedA"])
def test_grouped_repacked(orc, dtype, K, shift_a):
    """Grouped calls with rows that are not a multiple of 16 bytes, or an A
    off a 16-byte boundary: against the oracle, and bit for bit against the
    same call on host-padded operands."""
    G, total_m, N = 5, 700, 300
    offs = np.array([90, 90, 333, 600, 700], dtype=np.int32)   # one empty group
    A, _ = workloads.random_operands(dtype, total_m, 1, K, 1, seed=K)
    _, B = workloads.random_operands(dtype, 1, N, K, G, seed=K + 1)
    A = A[0]
    C = _grouped_run(A, B, offs, dtype, "relu", shift_a)
    ref = orc.gemm_grouped64(A, B, offs, dtype, "relu")
    assert_close(C, ref, A, B, dtype, K, f"grouped {dtype} K={K} shift_a={shift_a}")
    vec = 16 // EB[dtype]
    Kp = (K + vec - 1) // vec * vec
    Cpad = _grouped_run(_pad(A, Kp), _pad(B, Kp), offs, dtype, "relu")
    assert_bits_equal(C, Cpad, f"grouped {dtype} K={K} against host-padded")
