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


def _digest_table():
    out = {}
    with open(os.path.join(HERE, "golden", "full_int_digests.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, epi, l, m0, rows, h = line.split()
            out[(key, epi, int(l), int(m0))] = (int(rows), h)
    return out


def _exact_int_block_bits(A0, B0, m0, rows, epi, dtype):
    """Rows m0..m0+rows of one batch for integer-valued operands, computed
    without the oracle: every product and sum is an integer below 2^53, so a
    float64 BLAS matmul is exact; the integers (below 2^24) convert to float32
    exactly, and float32 -> fp16 / bf16 then rounds once (numpy / torch)."""
    import torch

    a = A0[m0:m0 + rows].astype(np.float64)
    c = a @ B0.astype(np.float64).T
    assert np.all(c == np.round(c)) and np.max(np.abs(c)) < 2 ** 24
    if epi == "relu":
        c = np.where(c > 0, c, 0.0)
    c32 = c.astype(np.float32)
    if dtype == "f16":
        return c32.astype(np.float16).view(np.uint16)
    return torch.from_numpy(c32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _widened(bits, dtype):
    import torch

    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def test_full_output_digests_pinned_by_exact_integer_products():
    """The stored digests of the two largest workloads (written by
    make_full_digests.py from the oracle) against blocks recomputed here with
    exact integer arithmetic: the first and last 64-row blocks of batch 0."""
    import hashlib

    from tiled_dense_gemm_mkl_amd import workloads

    table = _digest_table()
    for key, epi in (("f16_8192x8192x8192_identity", "identity"), ("bf16_L8_512x3584x18944_silu", "relu")):
        w = workloads.WORKLOADS[key]
        # batch 0 is the first pair of draws of the integer stream (seed + 100)
        A, B = workloads.random_operands(w.dtype, w.M, w.N, w.K, 1, w.seed + 100, w.dist_a, w.dist_b, True)
        A0, B0 = _widened(A[0], w.dtype), _widened(B[0], w.dtype)
        for m0 in (0, w.M - 64):
            rows, h = table[(key, epi, 0, m0)]
            bits = _exact_int_block_bits(A0, B0, m0, rows, epi, w.dtype)
            got = hashlib.sha256(bits.astype("<u2").tobytes()).hexdigest()[:32]
            assert got == h, f"{key} block {m0}: {got} != stored {h}"
