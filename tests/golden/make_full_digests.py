#!/usr/bin/env python3
"""Writes tests/golden/full_int_digests.txt: digests of the oracle's whole
result on the integer-valued inputs of the two largest workloads.

The oracle computes every output of

    C[l][m][n] = epilogue( sum_k A[l][m][k] * B[l][n][k] )

in binary64 and rounds it once to the output type.  With integer inputs in
[-2, 2] every sum is an integer of magnitude at most 4 K, which fp32 holds
exactly, so a correct GPU path reproduces these bits exactly.  The result is
too large to store (128 MB and 29 MB), so this script stores one SHA-256 per
block of ROWS output rows of each batch (the stored bits of the block,
row-major, little-endian), and the GPU tests hash their output the same way.

Only the oracle and the seeded input generator are called here; nothing of
the GPU path is imported.  Run from the repository root:

    python tests/golden/make_full_digests.py
"""
from __future__ import annotations

import hashlib
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

OUT = os.path.join(ROOT, "tests", "golden", "full_int_digests.txt")
ROWS = 64

# (workload key, epilogue): SiLU is never bit-exact (the two sides' exp
# differ), so the SiLU workload is checked bit for bit through ReLU.
CASES = [
    ("f16_8192x8192x8192_identity", "identity"),
    ("bf16_L8_512x3584x18944_silu", "relu"),
]


def block_digests(bits, rows: int = ROWS):
    """[(batch, first row, row count, hex digest)] of a [L, M, N] array of stored bits."""
    out = []
    L, M, _ = bits.shape
    for l in range(L):
        for m0 in range(0, M, rows):
            blk = bits[l, m0:m0 + rows]
            h = hashlib.sha256(blk.astype(blk.dtype.newbyteorder("<"), copy=False).tobytes()).hexdigest()[:32]
            out.append((l, m0, blk.shape[0], h))
    return out


def main() -> int:
    import oracle
    from tiled_dense_gemm_mkl_amd import workloads

    oracle.build(force=False)
    lines = [
        "# SHA-256 (first 32 hex digits) of the oracle's single-rounded output on the",
        "# integer-valued inputs (workloads.make_inputs(key, integer=True)), per block",
        f"# of {ROWS} rows of each batch: stored bits, row-major, little-endian.",
        "# Written by tests/golden/make_full_digests.py (oracle and input generator only).",
        "# key epilogue batch first_row rows digest",
    ]
    for key, epi in CASES:
        w = workloads.WORKLOADS[key]
        t0 = time.time()
        A, B = workloads.make_inputs(w, integer=True)
        y = oracle.gemm64(A, B, w.dtype, epi)
        bits = oracle.round_to_dtype(y, w.dtype)
        del y
        for l, m0, rows, h in block_digests(bits):
            lines.append(f"{key} {epi} {l} {m0} {rows} {h}")
        print(f"{key} {epi}: {time.time() - t0:.1f} s", flush=True)
    with open(OUT, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {OUT}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
