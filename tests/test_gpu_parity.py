"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Run on an MI355X:  python -u -m pytest tests -m gpu -x -v --timeout 120 --timeout-method thread
"""
from __future__ import annotations

import numpy as np
import pytest

import tiled_dense_gemm_mkl_amd as gm
from tiled_dense_gemm_mkl_amd import workloads
from gpu_helpers import (TOL, assert_bits_equal, assert_close, require_gpu, run_gemm,
                         to_device, widen_bits)

pytestmark = pytest.mark.gpu

DTYPES = ("f32", "f16", "bf16")
EPIS = ("identity", "relu", "silu")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _operands(dtype, M, N, K, L, seed, integer=False, dist=("uniform", -1.0, 1.0)):
    return workloads.random_operands(dtype, M, N, K, L, seed, dist, dist, integer)


# ---------------------------------------------------------------- small and ragged shapes, full check

RAGGED = [
    (1, 1, 8, 1),
    (5, 3, 8, 1),
    (17, 33, 40, 2),
    (64, 64, 64, 1),
    (129, 257, 136, 3),
    (200, 100, 328, 1),
    (300, 70, 1000, 2),
    (128, 128, 4096, 1),
]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
def test_ragged_shapes_all_epilogues(orc, dtype, shape):
    M, N, K, L = shape
    if dtype == "f32" and K % 4:
        pytest.skip("covered by the general-kernel test")
    A, B = _operands(dtype, M, N, K, L, seed=M * 7 + N * 3 + K)
    for epi in EPIS:
        ref = orc.gemm64(A, B, dtype, epi)
        C = run_gemm(A, B, dtype, epi)
        assert_close(C, ref, A, B, dtype, K, f"{dtype} {shape} {epi}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", [(33, 17, 13, 2), (70, 65, 37, 1), (5, 129, 3, 3), (64, 64, 1, 1)],
                         ids=lambda s: "x".join(map(str, s)))
def test_unaligned_K_repacked_and_general(orc, dtype, shape):
    """Rows that are not a multiple of 16 bytes: the automatic plan repacks A
    and B; the general kernel (forced) must agree with the oracle as well."""
    M, N, K, L = shape
    A, B = _operands(dtype, M, N, K, L, seed=K + 1)
    plan = gm.get_plan(M, N, K, L, gm.DTYPE_CODES[dtype], gm.EPI_RELU)
    if (K * (4 if dtype == "f32" else 2)) % 16:
        assert plan["packed"] == 1 and plan["general"] == 0
    for epi in EPIS:
        ref = orc.gemm64(A, B, dtype, epi)
        C = run_gemm(A, B, dtype, epi)
        assert_close(C, ref, A, B, dtype, K, f"repacked {dtype} {shape} {epi}")
        Cg = run_gemm(A, B, dtype, epi, force_general=True)
        assert_close(Cg, ref, A, B, dtype, K, f"general {dtype} {shape} {epi}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_general_kernel_forced_and_misaligned(orc, dtype):
    import torch

    M, N, K, L = 45, 77, 96, 2
    A, B = _operands(dtype, M, N, K, L, seed=99)
    ref = orc.gemm64(A, B, dtype, "silu")
    C = run_gemm(A, B, dtype, "silu", force_general=True)
    assert_close(C, ref, A, B, dtype, K, "forced general")
    # operands that start one element past a 16-byte boundary are repacked
    a_big = to_device(np.concatenate([A.reshape(-1)[:1], A.reshape(-1)]), dtype)
    b_big = to_device(np.concatenate([B.reshape(-1)[:1], B.reshape(-1)]), dtype)
    a = a_big[1:].view(L, M, K)
    b = b_big[1:].view(L, N, K)
    c = gm.gemm(a, b, "silu")
    torch.cuda.synchronize()
    assert_close(workloads.torch_to_storage(c), ref, A, B, dtype, K, "misaligned operands")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("epi", EPIS)
def test_K_zero_gives_epilogue_of_zero(dtype, epi):
    import torch

    st = np.float32 if dtype == "f32" else np.uint16
    A = np.zeros((2, 19, 0), st)
    B = np.zeros((2, 23, 0), st)
    a, b = to_device(A, dtype), to_device(B, dtype)
    c = torch.full((2, 19, 23), 7.0, dtype=a.dtype, device=a.device)
    gm.gemm(a, b, epi, out=c)
    torch.cuda.synchronize()
    assert torch.all(c == 0).item()


# ---------------------------------------------------------------- the five workloads

SMALL = ["f32_128x128x128_identity", "f32_128x2048x2048_relu"]


@pytest.mark.parametrize("key", SMALL)
def test_workload_full_parity(orc, key):
    w = workloads.WORKLOADS[key]
    A, B = workloads.make_inputs(w)
    ref = orc.gemm64(A, B, w.dtype, w.epilogue)
    C = run_gemm(A, B, w.dtype, w.epilogue)
    err = assert_close(C, ref, A, B, w.dtype, w.K, key)
    print(f"{key}: err {err:.3e} (tol {TOL[w.dtype]:.0e})")


@pytest.mark.parametrize("key", SMALL)
def test_workload_integer_inputs_bit_exact(orc, key):
    """Integer inputs in [-2, 2]: every fp32 partial sum is exact, so the GPU
    must reproduce the oracle's single rounding bit for bit.  (The three large
    workloads are checked in full in test_gpu_full_parity.py.)"""
    w = workloads.WORKLOADS[key]
    A, B = workloads.make_inputs(w, integer=True)
    epi = "relu" if w.epilogue == "silu" else w.epilogue
    C = run_gemm(A, B, w.dtype, epi)
    ref = orc.round_to_dtype(orc.gemm64(A, B, w.dtype, epi), w.dtype)
    assert_bits_equal(C, ref, key)


# ---------------------------------------------------------------- invariants

def _configs_of(dtype):
    return [i for i, n in enumerate(gm.config_names()) if n.split()[0] == dtype]


@pytest.mark.parametrize("dtype", DTYPES)
def test_prefetch_depth_does_not_change_results(orc, dtype):
    """The ring changes timing, never arithmetic: bitwise identical output for
    every prefetch depth a configuration provides (a race check)."""
    M, N, K, L = 300, 200, 2048 + 64, 2
    A, B = _operands(dtype, M, N, K, L, seed=123)
    ref = orc.gemm64(A, B, dtype, "identity")
    for cid in _configs_of(dtype):
        outs = {}
        sk_outs = {}
        for p in range(0, 9):
            try:
                sk = gm.get_plan(M, N, K, L, gm.DTYPE_CODES[dtype], gm.EPI_IDENTITY,
                                 gm.make_opts(config_id=cid, prefetch_stages=p, streamk=True))
            except gm.GemmMklError:
                sk = None
            if sk is not None:
                assert sk["streamk"] == 1
                sk_outs[p] = run_gemm(A, B, dtype, "identity", config_id=cid, prefetch_stages=p, streamk=True)
            try:
                gm.get_plan(M, N, K, L, gm.DTYPE_CODES[dtype], gm.EPI_IDENTITY,
                            gm.make_opts(config_id=cid, prefetch_stages=p, split_k=1))
            except gm.GemmMklError:
                continue
            outs[p] = run_gemm(A, B, dtype, "identity", config_id=cid, prefetch_stages=p, split_k=1)
        assert len(outs) >= 1
        first = next(iter(outs.values()))
        assert_close(first, ref, A, B, dtype, K, f"config {cid}")
        for p, C in outs.items():
            assert_bits_equal(C, first, f"config {cid} prefetch {p}")
        if sk_outs:
            sk_first = next(iter(sk_outs.values()))
            assert_close(sk_first, ref, A, B, dtype, K, f"config {cid} stream-K")
            for p, C in sk_outs.items():
                assert_bits_equal(C, sk_first, f"config {cid} stream-K prefetch {p}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_every_config_and_split(orc, dtype):
    M, N, K, L = 270, 390, 1536 + 8 * (2 if dtype != "f32" else 1), 2
    A, B = _operands(dtype, M, N, K, L, seed=321)
    ref = orc.gemm64(A, B, dtype, "relu")
    Ai, Bi = _operands(dtype, M, N, K, L, seed=322, integer=True)
    refi = orc.round_to_dtype(orc.gemm64(Ai, Bi, dtype, "identity"), dtype)
    for cid in _configs_of(dtype):
        for S in (1, 2, 3, 5):
            C = run_gemm(A, B, dtype, "relu", config_id=cid, split_k=S)
            assert_close(C, ref, A, B, dtype, K, f"config {cid} S={S}")
            Ci = run_gemm(Ai, Bi, dtype, "identity", config_id=cid, split_k=S)
            assert_bits_equal(Ci, refi, f"integer config {cid} S={S}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_relu_is_max_of_identity_and_batches_are_independent(dtype):
    import torch

    M, N, K, L = 160, 260, 512, 3
    A, B = _operands(dtype, M, N, K, L, seed=7)
    a, b = to_device(A, dtype), to_device(B, dtype)
    # one fixed plan for every call: results depend on the tile configuration
    # and the split (summation order), not on the batch count
    plan = gm.get_plan(M, N, K, L, gm.DTYPE_CODES[dtype], gm.EPI_IDENTITY)
    fixed = dict(config_id=plan["config_id"], split_k=plan["split_k"], prefetch_stages=plan["prefetch_stages"])
    c_id = gm.gemm(a, b, "identity", **fixed)
    c_relu = gm.gemm(a, b, "relu", **fixed)
    torch.cuda.synchronize()
    want = torch.where(c_id > 0, c_id, torch.zeros_like(c_id))
    assert_bits_equal(workloads.torch_to_storage(c_relu), workloads.torch_to_storage(want), "relu vs identity")
    for l in range(L):
        one = gm.gemm(a[l:l + 1].contiguous(), b[l:l + 1].contiguous(), "identity", **fixed)
        torch.cuda.synchronize()
        assert_bits_equal(workloads.torch_to_storage(one[0]), workloads.torch_to_storage(c_id[l]),
                          f"batch {l}")
    # run-to-run determinism of the automatic plan
    again = gm.gemm(a, b, "identity", **fixed)
    torch.cuda.synchronize()
    assert_bits_equal(workloads.torch_to_storage(again), workloads.torch_to_storage(c_id), "rerun")


@pytest.mark.parametrize("dtype", DTYPES)
def test_guard_bands_untouched(dtype):
    """Canaries before and after C, and after the caller's workspace."""
    import torch

    M, N, K, L = 130, 70, 264, 2
    A, B = _operands(dtype, M, N, K, L, seed=11)
    a, b = to_device(A, dtype), to_device(B, dtype)
    tdt = a.dtype
    pad = 4096
    buf = torch.full((pad + L * M * N + pad,), 1234.0, dtype=tdt, device=a.device)
    out = buf[pad:pad + L * M * N].view(L, M, N)
    ws_need = gm.get_plan(M, N, K, L, gm.DTYPE_CODES[dtype], gm.EPI_SILU, gm.make_opts(split_k=3))["workspace_bytes"]
    ws = torch.full((ws_need // 4 + pad,), -5.0, dtype=torch.float32, device=a.device)
    gm.gemm(a, b, "silu", out=out, split_k=3, workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(buf[:pad] == 1234.0).item() and torch.all(buf[-pad:] == 1234.0).item()
    assert torch.all(ws[ws_need // 4:] == -5.0).item()
    ref = gm.gemm(a, b, "silu", split_k=3)
    torch.cuda.synchronize()
    assert_bits_equal(workloads.torch_to_storage(out), workloads.torch_to_storage(ref), "caller vs internal workspace")


def test_operands_end_to_end_in_one_buffer():
    """A, B and C laid end to end in one allocation share no byte: the call
    runs and equals the call on separate tensors bit for bit.  A C over A is
    refused (INVALID_VALUE) before any launch, and A is left as it was."""
    import torch

    M, N, K, L = 96, 80, 128, 2
    A, B = _operands("bf16", M, N, K, L, seed=21)
    a, b = to_device(A, "bf16"), to_device(B, "bf16")
    na, nb, nc = a.numel(), b.numel(), L * M * N
    buf = torch.empty(na + nb + nc, dtype=a.dtype, device=a.device)
    buf[:na] = a.flatten()
    buf[na:na + nb] = b.flatten()
    a2, b2, c2 = buf[:na].view(L, M, K), buf[na:na + nb].view(L, N, K), buf[na + nb:].view(L, M, N)
    gm.gemm(a2, b2, "relu", out=c2)
    ref = gm.gemm(a, b, "relu")
    torch.cuda.synchronize()
    assert_bits_equal(workloads.torch_to_storage(c2), workloads.torch_to_storage(ref), "one buffer vs separate")
    with pytest.raises(gm.GemmMklError) as e:
        gm.gemm(a2, b2, "relu", out=buf[:nc].view(L, M, N))
    assert e.value.status == -1
    torch.cuda.synchronize()
    assert torch.equal(a2, a)


def test_workspace_too_small_is_rejected_and_C_untouched():
    import torch

    M, N, K, L = 128, 128, 1024, 1
    A, B = _operands("bf16", M, N, K, L, seed=3)
    a, b = to_device(A, "bf16"), to_device(B, "bf16")
    c = torch.full((L, M, N), 3.0, dtype=a.dtype, device=a.device)
    ws = torch.zeros(16, dtype=torch.float32, device=a.device)
    with pytest.raises(gm.GemmMklError) as e:
        gm.gemm(a, b, "relu", out=c, split_k=2, workspace=ws)
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert torch.all(c == 3.0).item()
    # a workspace in host memory is refused before any launch
    with pytest.raises(ValueError, match="workspace"):
        gm.gemm(a, b, "relu", out=c, split_k=2, workspace=torch.zeros(1 << 20))
    torch.cuda.synchronize()
    assert torch.all(c == 3.0).item()


def test_non_default_stream(orc):
    import torch

    M, N, K, L = 256, 256, 512, 1
    A, B = _operands("bf16", M, N, K, L, seed=17)
    ref = orc.gemm64(A, B, "bf16", "relu")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        a, b = to_device(A, "bf16"), to_device(B, "bf16")
        c = gm.gemm(a, b, "relu")
    s.synchronize()
    assert_close(workloads.torch_to_storage(c), ref, A, B, "bf16", K, "side stream")


def test_raw_c_abi_entry_point(orc):
    """gemm_mkl itself (not _ex), with raw device pointers and a null stream."""
    import torch

    M, N, K, L = 96, 80, 192, 2
    A, B = _operands("f16", M, N, K, L, seed=5)
    a, b = to_device(A, "f16"), to_device(B, "f16")
    c = torch.empty((L, M, N), dtype=a.dtype, device=a.device)
    torch.cuda.synchronize()
    st = gm.gemm_mkl(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, L, gm.F16, gm.EPI_SILU, None)
    assert st == 0, gm.status_string(st)
    torch.cuda.synchronize()
    assert_close(workloads.torch_to_storage(c), orc.gemm64(A, B, "f16", "silu"), A, B, "f16", K, "raw ABI")


# ---------------------------------------------------------------- stream-K

SK_SHAPES = [(300, 390, 1552, 2), (512, 640, 2048, 1), (129, 257, 1000, 3), (64, 64, 4096, 1)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", SK_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_streamk_parity_and_determinism(orc, dtype, shape):
    """Stream-K (forced): oracle parity, integer inputs bit-exact, and the same
    bits on every run (the fix-up sums pieces in a fixed order)."""
    M, N, K, L = shape
    code = gm.DTYPE_CODES[dtype]
    try:
        plan = gm.get_plan(M, N, K, L, code, gm.EPI_SILU, gm.make_opts(streamk=True))
    except gm.GemmMklError as e:
        assert e.status == -6
        pytest.skip("no stream-K configuration fits this shape")
    assert plan["streamk"] == 1 and plan["grid"] <= 256
    A, B = _operands(dtype, M, N, K, L, seed=K + 7)
    ref = orc.gemm64(A, B, dtype, "silu")
    C1 = run_gemm(A, B, dtype, "silu", streamk=True)
    assert_close(C1, ref, A, B, dtype, K, f"stream-K {dtype} {shape}")
    C2 = run_gemm(A, B, dtype, "silu", streamk=True)
    assert_bits_equal(C1, C2, "stream-K run-to-run")
    Ai, Bi = _operands(dtype, M, N, K, L, seed=K + 8, integer=True)
    refi = orc.round_to_dtype(orc.gemm64(Ai, Bi, dtype, "relu"), dtype)
    assert_bits_equal(run_gemm(Ai, Bi, dtype, "relu", streamk=True), refi, f"stream-K integer {dtype} {shape}")


def test_streamk_caller_workspace_counters_return_to_zero(orc):
    import torch

    M, N, K, L = 512, 640, 2048, 1
    A, B = _operands("bf16", M, N, K, L, seed=31)
    a, b = to_device(A, "bf16"), to_device(B, "bf16")
    plan = gm.get_plan(M, N, K, L, gm.BF16, gm.EPI_RELU, gm.make_opts(streamk=True))
    assert plan["streamk"] == 1 and plan["counter_bytes"] > 0
    ws = torch.zeros(plan["workspace_bytes"] // 4 + 1024, dtype=torch.float32, device=a.device)
    outs = []
    for _ in range(3):
        outs.append(gm.gemm(a, b, "relu", streamk=True, workspace=ws))
        torch.cuda.synchronize()
        assert torch.all(ws[: plan["counter_bytes"] // 4] == 0).item(), "counters left non-zero"
    internal = gm.gemm(a, b, "relu", streamk=True)
    torch.cuda.synchronize()
    for o in outs:
        assert_bits_equal(workloads.torch_to_storage(o), workloads.torch_to_storage(internal), "caller ws")
    assert_close(workloads.torch_to_storage(internal), orc.gemm64(A, B, "bf16", "relu"), A, B, "bf16", K, "sk")


def test_streamk_and_split_k_exclude_each_other():
    with pytest.raises(gm.GemmMklError) as e:
        gm.get_plan(512, 640, 2048, 1, gm.BF16, gm.EPI_RELU, gm.make_opts(streamk=True, split_k=2))
    assert e.value.status == -6
