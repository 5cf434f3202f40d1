"""The oracle against small hand-worked fixtures under tests/golden/."""
import os

import numpy as np

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _read(name):
    rows = []
    with open(os.path.join(HERE, "golden", name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(v) for v in line.split()])
    return rows


def test_handworked_int_gemm(orc):
    rows = _read("handworked_int_gemm.txt")
    L, M, N, K = rows[0]
    it = iter(rows[1:])
    A = np.array([next(it) for _ in range(L * M)], np.float64).reshape(L, M, K)
    B = np.array([next(it) for _ in range(L * N)], np.float64).reshape(L, N, K)
    C_id = np.array([next(it) for _ in range(L * M)], np.float64).reshape(L, M, N)
    C_relu = np.array([next(it) for _ in range(L * M)], np.float64).reshape(L, M, N)
    for dtype in ("f32", "f16", "bf16"):
        if dtype == "f32":
            a, b = A.astype(np.float32), B.astype(np.float32)
        else:
            a = orc.round_to_dtype(A, dtype)
            b = orc.round_to_dtype(B, dtype)
        assert np.array_equal(orc.gemm64(a, b, dtype, "identity"), C_id)
        got = orc.gemm64(a, b, dtype, "relu")
        assert np.array_equal(got, C_relu) and not np.any(np.signbit(got))
