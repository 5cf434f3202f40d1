"""The C-ABI calls captured in a HIP graph: every replay, with eager work and
synchronisations between replays, gives the eager result bit for bit (the
headline GEMM, a split-K GEMM with its reduction kernel, and the RMSNorm)."""
import numpy as np
import pytest

import tiled_dense_gemm_mkl_amd as gm
from tiled_dense_gemm_mkl_amd import workloads
from gpu_helpers import assert_bits_equal, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _check_graph(call, out, replays=4):
    import torch

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        call(stream.cuda_stream)            # eager (also allocates any workspace)
    torch.cuda.synchronize()
    eager = workloads.torch_to_storage(out).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        call(stream.cuda_stream)
    for r in range(replays):
        out.fill_(0)                        # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_bits_equal(workloads.torch_to_storage(out), eager, f"replay {r}")
        with torch.cuda.stream(stream):
            call(stream.cuda_stream)        # and an eager call again
        torch.cuda.synchronize()


def test_graph_headline_gemm():
    w = workloads.WORKLOADS[workloads.HEADLINE]
    A, B = workloads.make_inputs(w)
    a = workloads.storage_to_torch(A, w.dtype).cuda()
    b = workloads.storage_to_torch(B, w.dtype).cuda()
    import torch

    c = torch.empty((w.L, w.M, w.N), dtype=a.dtype, device="cuda")
    _check_graph(lambda s: gm.gemm_mkl(a.data_ptr(), b.data_ptr(), c.data_ptr(), w.M, w.N, w.K, w.L,
                                       gm.BF16, gm.EPI_RELU, s), c)


def test_graph_split_k_gemm():
    import torch

    w = workloads.WORKLOADS["f32_128x2048x2048_relu"]
    A, B = workloads.make_inputs(w)
    a = workloads.storage_to_torch(A, w.dtype).cuda()
    b = workloads.storage_to_torch(B, w.dtype).cuda()
    c = torch.empty((w.L, w.M, w.N), dtype=a.dtype, device="cuda")
    assert gm.get_plan(w.M, w.N, w.K, w.L, gm.F32, gm.EPI_RELU)["split_k"] > 1
    _check_graph(lambda s: gm.gemm_mkl(a.data_ptr(), b.data_ptr(), c.data_ptr(), w.M, w.N, w.K, w.L,
                                       gm.F32, gm.EPI_RELU, s), c)


def test_graph_rms_norm():
    import torch

    X, W = workloads.make_rms_inputs("rmsnorm_f32_32x2048")
    x = torch.from_numpy(X).cuda()
    wt = torch.from_numpy(W).cuda()
    y = torch.empty_like(x)
    _check_graph(lambda s: gm.gemm_mkl_rms_norm(x.data_ptr(), wt.data_ptr(), y.data_ptr(), 32, 2048, 1e-6,
                                                gm.F32, s), y)
