"""GPU tests of split-K with the in-kernel fix-up (the S pieces of a tile run on
one XCD and the last one to finish sums them in ascending split order).

The fix-up computes the same partials in the same order as the split-K grid
with the separate reduction kernel, so the two must agree bit for bit; both are
checked against the oracle (random inputs within the tolerance, integer inputs
bit for bit).  The path where the last piece recomputes the other pieces
itself (taken when a partial was written on another XCD) is forced from the
host and must give the same bits too.
"""
from __future__ import annotations

import pytest

import tiled_dense_gemm_mkl_amd as gm
from tiled_dense_gemm_mkl_amd import workloads
from gpu_helpers import assert_bits_equal, assert_close, require_gpu, run_gemm, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _cid(name):
    return gm.config_names().index(name)


CASES = [
    # (dtype, M, N, K, L, split, configuration)
    ("bf16", 512, 5632, 2048, 1, 2, "bf16 128x192 k64 waves2x2+4p mfma32"),
    ("bf16", 300, 500, 1000, 2, 3, "bf16 128x192 k64 waves2x2+4p mfma32"),
    ("f16", 260, 390, 1544, 1, 2, "f16 128x192 k64 waves2x2+4p mfma32"),
    ("bf16", 270, 390, 1552, 2, 4, "bf16 128x128 k64 waves2x2+4p mfma32"),
    ("f16", 129, 257, 2048, 1, 6, "f16 128x128 k64 waves2x2+4p mfma32"),
    ("bf16", 300, 520, 4096, 1, 2, "bf16 256x256 k32 waves2x2 mfma32"),
    ("bf16", 512, 5632, 2048, 1, 2, "bf16 128x256 k64 waves2x2+4p mfma32"),
    ("f16", 300, 700, 1552, 2, 3, "f16 128x256 k64 waves2x2+4p mfma32"),
    ("bf16", 520, 390, 2048, 1, 2, "bf16 256x128 k64 waves2x2+4p mfma32"),
    ("bf16", 260, 600, 1040, 1, 4, "bf16 128x256 k32 waves2x2+4p mfma32"),
    ("f32", 128, 2048, 2048, 1, 4, "f32 64x64 k32 waves2x2 mfma16"),
    ("f32", 100, 300, 520, 3, 3, "f32 64x64 k32 waves2x2 mfma16"),
    ("f32", 200, 200, 1024, 1, 2, "f32 128x128 k32 waves2x2 mfma32"),
    ("f32", 128, 2048, 2048, 1, 4, "f32 64x64 k32 waves2x2+4p mfma16"),
    ("f32", 100, 300, 520, 3, 3, "f32 64x64 k32 waves2x2+4p mfma16"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}x{c[4]}-S{c[5]}-{c[6].split()[1]}")
def test_fixup_equals_split_k_reduction_and_oracle(orc, case):
    dtype, M, N, K, L, S, cfg = case
    kw = dict(config_id=_cid(cfg), split_k=S)
    plan = gm.get_plan(M, N, K, L, gm.DTYPE_CODES[dtype], gm.EPI_SILU, gm.make_opts(fixup=True, **kw))
    assert plan["fixup"] == 1 and plan["split_k"] == S
    A, B = workloads.random_operands(dtype, M, N, K, L, seed=M + N + K + S)
    fix = run_gemm(A, B, dtype, "silu", fixup=True, **kw)
    red = run_gemm(A, B, dtype, "silu", fixup=False, **kw)
    assert_bits_equal(fix, red, f"fix-up vs reduction kernel {case}")
    again = run_gemm(A, B, dtype, "silu", fixup=True, **kw)
    assert_bits_equal(again, fix, f"fix-up run-to-run {case}")
    rec = run_gemm(A, B, dtype, "silu", fixup=True, fixup_recompute=True, **kw)
    assert_bits_equal(rec, fix, f"fix-up with every other piece recomputed {case}")
    assert_close(fix, orc.gemm64(A, B, dtype, "silu"), A, B, dtype, K, f"fix-up {case}")
    Ai, Bi = workloads.random_operands(dtype, M, N, K, L, seed=M + N + K + S + 1, integer=True)
    ref = orc.round_to_dtype(orc.gemm64(Ai, Bi, dtype, "relu"), dtype)
    assert_bits_equal(run_gemm(Ai, Bi, dtype, "relu", fixup=True, **kw), ref, f"fix-up integer {case}")
    assert_bits_equal(run_gemm(Ai, Bi, dtype, "relu", fixup=True, fixup_recompute=True, **kw), ref,
                      f"fix-up recomputed integer {case}")


def test_fixup_caller_workspace_counters_return_to_zero(orc):
    import torch

    M, N, K, L = 512, 5632, 2048, 1
    cfg = _cid("bf16 128x192 k64 waves2x2+4p mfma32")
    o = gm.make_opts(split_k=2, config_id=cfg, fixup=True)
    plan = gm.get_plan(M, N, K, L, gm.BF16, gm.EPI_RELU, o)
    assert plan["fixup"] == 1 and plan["counter_bytes"] > 0
    A, B = workloads.random_operands("bf16", M, N, K, L, seed=77, dist_a=("normal", 1.0), dist_b=("normal", 0.02))
    a, b = to_device(A, "bf16"), to_device(B, "bf16")
    ws = torch.zeros(plan["workspace_bytes"] // 4 + 64, dtype=torch.float32, device=a.device)
    outs = []
    for recompute in (False, True, False):
        outs.append(gm.gemm(a, b, "relu", split_k=2, config_id=cfg, fixup=True, fixup_recompute=recompute,
                            workspace=ws))
        torch.cuda.synchronize()
        assert torch.all(ws[: plan["counter_bytes"] // 4] == 0).item(), "counters left non-zero"
    for c in outs[1:]:
        assert_bits_equal(workloads.torch_to_storage(c), workloads.torch_to_storage(outs[0]), "caller workspace")
    internal = gm.gemm(a, b, "relu", split_k=2, config_id=cfg, fixup=True)
    torch.cuda.synchronize()
    assert_bits_equal(workloads.torch_to_storage(internal), workloads.torch_to_storage(outs[0]), "internal workspace")
    assert_close(workloads.torch_to_storage(internal), orc.gemm64(A, B, "bf16", "relu"), A, B, "bf16", K, "fix-up")


def test_fixup_through_noalloc(orc):
    """The allocation-free entry point keeps the fix-up's counters in the tail
    of its scratch: two calls in a row, then a non-fix-up split call that
    writes partials into the scratch, then the fix-up again."""
    import torch

    A, B = workloads.random_operands("f32", 128, 2048, 2048, 1, seed=3)
    a, b = to_device(A, "f32"), to_device(B, "f32")
    ref = orc.gemm64(A, B, "f32", "relu")
    s = torch.cuda.current_stream().cuda_stream
    outs = []
    for fx in (True, True, False, True):
        c = torch.empty((1, 128, 2048), dtype=torch.float32, device=a.device)
        st = gm.gemm_mkl_noalloc(a.data_ptr(), b.data_ptr(), c.data_ptr(), 128, 2048, 2048, 1, gm.F32, gm.EPI_RELU, s,
                                 gm.make_opts(split_k=4, config_id=_cid("f32 64x64 k32 waves2x2 mfma16"), fixup=fx))
        assert st == 0, gm.status_string(st)
        torch.cuda.synchronize()
        outs.append(workloads.torch_to_storage(c))
    for c in outs:
        assert_bits_equal(c, outs[0], "noalloc fix-up / reduction")
    assert_close(outs[0], ref, A, B, "f32", 2048, "noalloc fix-up")
