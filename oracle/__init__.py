"""CPU oracle for the batched "mkl" GEMM with a fused epilogue, the grouped
GEMM, and the RMSNorm row reduction.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this package.  The product path (the HIP
library and its Python binding) never imports, loads or calls it, and the two
share no code: this package does not import the product package either.

The arithmetic lives in ``gemm_oracle.c`` (plain C, binary64 accumulation, one
rounding to the output type); this module only builds it, loads it with ctypes
and marshals numpy arrays.
"""
from .oracle import (  # noqa: F401
    DTYPES,
    EPILOGUES,
    build,
    epilogue64,
    gemm64,
    gemm_entries64,
    gemm_grouped64,
    gemm_rounded,
    load,
    rms_norm64,
    round_to_dtype,
    threads,
    widen,
)
