"""Calls from several host threads at once, each on its own stream.

The library keeps one plan cache for the process and one split-K / stream-K
workspace per (device, stream), both behind mutexes.  Four threads run a mix
of plans (split-K with the library's workspace, forced stream-K with its
counters, a single-pass tile grid, a grouped GEMM) on their own streams, each
many times; every result must equal the same call made alone, bit for bit
(each plan is deterministic)."""
import threading

import numpy as np
import pytest

import tiled_dense_gemm_mkl_amd as gm
from tiled_dense_gemm_mkl_amd import workloads
from gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu

CASES = [  # (dtype, M, N, K, L, opts kwargs)
    ("f32", 128, 2048, 2048, 1, {}),                   # automatic split-K + reduce
    ("bf16", 1000, 1100, 520, 1, {"streamk": True}),   # stream-K: counters per stream
    ("bf16", 512, 5632, 2048, 1, {}),                  # producer configuration, one pass
    ("f16", 300, 700, 2000, 2, {"split_k": 3}),        # forced split with batches
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _inputs(i, dtype, M, N, K, L):
    import torch

    A, B = workloads.random_operands(dtype, M, N, K, L, seed=500 + i)
    a = workloads.storage_to_torch(A, dtype).cuda()
    b = workloads.storage_to_torch(B, dtype).cuda()
    c = torch.empty((L, M, N), dtype=a.dtype, device="cuda")
    return a, b, c


def _call(a, b, c, dtype, M, N, K, L, kw, stream):
    st = gm.gemm_mkl_ex(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, L, gm.DTYPE_CODES[dtype],
                        gm.EPI_RELU, stream.cuda_stream, gm.make_opts(**kw) if kw else None)
    assert st == 0, gm.status_string(st)


def test_threads_on_their_own_streams_match_serial_calls():
    import torch

    bufs = [_inputs(i, *case[:5]) for i, case in enumerate(CASES)]
    solo = []
    s0 = torch.cuda.Stream()
    for (dtype, M, N, K, L, kw), (a, b, c) in zip(CASES, bufs):
        _call(a, b, c, dtype, M, N, K, L, kw, s0)
        s0.synchronize()
        solo.append(c.clone())
    errors = []
    outs = [[] for _ in CASES]

    def worker(i):
        try:
            dtype, M, N, K, L, kw = CASES[i]
            a, b, _ = bufs[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(25):
                    c = torch.empty((L, M, N), dtype=a.dtype, device="cuda")
                    _call(a, b, c, dtype, M, N, K, L, kw, s)
                    outs[i].append(c)
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(CASES))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i, case in enumerate(CASES):
        assert len(outs[i]) == 25
        for r, c in enumerate(outs[i]):
            assert torch.equal(c.view(torch.int16 if c.element_size() == 2 else torch.int32),
                               solo[i].view(torch.int16 if c.element_size() == 2 else torch.int32)), \
                f"case {case}, repeat {r}: differs from the call made alone"
