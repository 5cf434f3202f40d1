"""Every tile configuration of the table on a seeded random ragged shape of its
own (M and N from 1 to 600, K a multiple of 8 up to 1600, one or two
batches): integer inputs through the data-parallel grid at the
configuration's own prefetch depth, and, where the configuration carries an
in-kernel fix-up kernel, through two K splits summed in the kernel; each
output bit for bit against the oracle's rounded result (integer products and
sums are exact in fp32 accumulation, so every correct order gives the same
bits)."""
import numpy as np
import pytest

import tiled_dense_gemm_mkl_amd as gm
from tiled_dense_gemm_mkl_amd import workloads
from gpu_helpers import assert_bits_equal, require_gpu, run_gemm

pytestmark = pytest.mark.gpu

CONFIGS = list(enumerate(gm.config_names()))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _shape(cid):
    rng = np.random.default_rng(7000 + cid)
    M, N = (int(v) for v in rng.integers(1, 601, 2))
    K = 8 * int(rng.integers(1, 201))
    L = int(rng.integers(1, 3))
    return M, N, K, L


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: f"{c[0]}-{c[1].replace(' ', '_')}")
def test_every_config_random_ragged_shape_integer_bit_exact(orc, cfg):
    cid, name = cfg
    dtype = name.split()[0]
    M, N, K, L = _shape(cid)
    print(f"config {cid} ({name}) at {M}x{N}x{K}x{L}", flush=True)
    code = gm.DTYPE_CODES[dtype]
    plan = gm.get_plan(M, N, K, L, code, gm.EPI_RELU, gm.make_opts(config_id=cid, split_k=1))
    assert plan["config_id"] == cid and plan["split_k"] == 1 and plan["general"] == 0
    A, B = workloads.random_operands(dtype, M, N, K, L, 7100 + cid, ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0),
                                     integer=True)
    ref = orc.round_to_dtype(orc.gemm64(A, B, dtype, "relu"), dtype)
    assert_bits_equal(run_gemm(A, B, dtype, "relu", config_id=cid, split_k=1), ref, f"{name} {M}x{N}x{K}x{L}")
    try:
        fp = gm.get_plan(M, N, K, L, code, gm.EPI_RELU, gm.make_opts(config_id=cid, split_k=2, fixup=True))
    except gm.GemmMklError as e:
        assert e.status == -6   # no fix-up kernel for this configuration
        return
    assert fp["fixup"] == 1 and fp["split_k"] == 2
    assert_bits_equal(run_gemm(A, B, dtype, "relu", config_id=cid, split_k=2, fixup=True), ref,
                      f"{name} {M}x{N}x{K}x{L} two pieces in the kernel")
