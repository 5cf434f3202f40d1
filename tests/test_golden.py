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


def test_handworked_rms_norm(orc):
    """RMSNorm against hand-worked closed forms (tests/golden/handworked_rms_norm.txt):
    binary64 within 4 units in the last place, for every storage type (the
    inputs are exact in all three)."""
    with open(os.path.join(HERE, "golden", "handworked_rms_norm.txt")) as f:
        lines = [l.split() for l in f if l.strip() and not l.startswith("#")]
    i, cases = 0, 0
    while i < len(lines):
        assert lines[i][0] == "case"
        rows, hidden, eps = int(lines[i][1]), int(lines[i][2]), float(lines[i][3])
        x = np.array([[float(v) for v in lines[i + 1 + r]] for r in range(rows)])
        w = np.array([float(v) for v in lines[i + 1 + rows]])
        y = np.array([[float(v) for v in lines[i + 2 + rows + r]] for r in range(rows)])
        assert x.shape == (rows, hidden) and w.shape == (hidden,) and y.shape == (rows, hidden)
        for dtype in ("f32", "f16", "bf16"):
            got = orc.rms_norm64(orc.round_to_dtype(x, dtype), orc.round_to_dtype(w, dtype), eps, dtype)
            assert np.all(np.abs(got - y) <= 4 * 2.0 ** -52 * np.abs(y)), (dtype, got, y)
        i += 2 + 2 * rows
        cases += 1
    assert cases == 5
