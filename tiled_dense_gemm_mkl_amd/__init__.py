"""MI355X-native tiled dense GEMM in the batched "mkl" layout.

    C[l][m][n] = epilogue( sum_k A[l][m][k] * B[l][n][k] )

A second kernel normalises rows (RMSNorm, ``rms_norm``).  The computation
runs in hand-written gfx950 HIP kernels behind the C ABI of
``include/gemm_mkl.h`` (``lib/libgemm_mkl.so``); this package is the thin
Python binding (argument marshalling only).  PyTorch supplies device memory
and streams.
"""
from ._binding import (  # noqa: F401
    BF16,
    DTYPE_CODES,
    EPI_IDENTITY,
    EPI_RELU,
    EPI_SILU,
    EPILOGUE_CODES,
    EXPORTS,
    F16,
    F32,
    LIB_PATH,
    STATUS,
    GemmMklError,
    config_names,
    gemm,
    gemm_grouped,
    gemm_mkl,
    gemm_mkl_ex,
    gemm_mkl_noalloc,
    NOALLOC_SCRATCH_BYTES,
    gemm_mkl_grouped,
    gemm_mkl_rms_norm,
    get_plan,
    tile_order,
    grouped_config,
    load,
    make_opts,
    release_workspace,
    rms_norm,
    rms_norm_variant,
    rms_norm_variant_names,
    status_string,
    workspace_size,
)
