"""GPU parity of the RMSNorm kernels (gemm_mkl_rms_norm) against the CPU oracle.

The GPU sums squares, takes the reciprocal square root and multiplies in fp32,
then rounds once to the storage type; the oracle does the same steps in
binary64.  Every output element must satisfy

    |y_gpu - y64| <= rel * |y64| + floor

with rel = 2^-17 for fp32 (the fp32 sum of a row's squares, the rsqrt and two
products stay far inside 128 units in the last place, for rows of up to 2^15
elements), and for fp16/bf16 half an output ulp on top (2^-11 resp. 2^-8
relative, plus half the smallest subnormal as the floor).  Rows scaled down to
1e-4 make eps the larger term under the square root, so a misplaced eps shows.
"""
import numpy as np
import pytest

import tiled_dense_gemm_mkl_amd as gm
from tiled_dense_gemm_mkl_amd import workloads
from gpu_helpers import assert_bits_equal, require_gpu, widen_bits

pytestmark = pytest.mark.gpu

DTYPES = ("f32", "f16", "bf16")
REL = {"f32": 2.0 ** -17, "f16": 2.0 ** -11 + 2.0 ** -17, "bf16": 2.0 ** -8 + 2.0 ** -17}
FLOOR = {"f32": 2.0 ** -149, "f16": 2.0 ** -25, "bf16": 2.0 ** -134}
EPS = 1e-6


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _vec_elems(dtype):
    return 4 if dtype == "f32" else 8


def _coverage(name, dtype):
    """Row length a vector variant covers ('vec nvX wY'), None for the general kernel."""
    if name == "general":
        return None
    nv, w = name.split()[1:]
    return int(nv[2:]) * int(w[1:]) * 64 * _vec_elems(dtype)


def _inputs(dtype, rows, hidden, seed, small_rows=0, weight=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, hidden))
    x[:small_rows] *= 1e-4
    w = 1.0 + 0.5 * rng.standard_normal(hidden) if weight else None
    X = workloads.to_storage(x, dtype)
    W = workloads.to_storage(w, dtype) if weight else None
    return X, W


def _run(X, W, dtype, eps=EPS, variant=-1, in_place=False, offset=0):
    """Upload, normalise on the GPU, download.  offset > 0 places x and y that
    many elements past a 256-byte boundary (not 16-byte aligned)."""
    import torch

    rows, hidden = X.shape
    if offset:
        flat = np.zeros(rows * hidden + offset, X.dtype)
        flat[offset:] = X.ravel()
        base = workloads.storage_to_torch(flat, dtype).cuda()
        x = base[offset:].view(rows, hidden)
        ybase = torch.empty_like(base)
        out = ybase[offset:].view(rows, hidden)
    else:
        x = workloads.storage_to_torch(np.ascontiguousarray(X), dtype).cuda()
        out = x if in_place else None
    w = workloads.storage_to_torch(np.ascontiguousarray(W), dtype).cuda() if W is not None else None
    y = gm.rms_norm(x, w, eps, out=out, variant=variant)
    torch.cuda.synchronize()
    return workloads.torch_to_storage(y)


def _ref(orc, X, W, dtype, eps=EPS):
    if W is None:
        ones = workloads.to_storage(np.ones(X.shape[1]), dtype)
        return orc.rms_norm64(X, ones, eps, dtype)
    return orc.rms_norm64(X, W, eps, dtype)


def _check(Y, y64, dtype, what):
    got = widen_bits(Y, dtype)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    bad = np.abs(got - y64) > REL[dtype] * np.abs(y64) + FLOOR[dtype]
    if bad.any():
        i = np.argmax(np.abs(got - y64) / (np.abs(y64) + FLOOR[dtype]))
        r, c = np.unravel_index(i, y64.shape)
        pytest.fail(f"{what}: {int(bad.sum())} elements off; worst at ({r},{c}): gpu {got[r, c]!r} "
                    f"oracle {y64[r, c]!r}")


HIDDEN = {"f32": [4, 260, 2048, 3000], "f16": [8, 264, 2048, 3584], "bf16": [8, 264, 2048, 3584]}


@pytest.mark.parametrize("dtype", DTYPES)
def test_rms_norm_parity_every_variant(orc, dtype):
    """Every variant that fits, on rows that do not fill the last workgroup
    (37), ragged last vectors, and rows small enough for eps to dominate."""
    names = gm.rms_norm_variant_names()
    for hidden in HIDDEN[dtype]:
        X, W = _inputs(dtype, 37, hidden, seed=hidden, small_rows=3)
        ref = _ref(orc, X, W, dtype)
        ran = 0
        for v, name in enumerate(names):
            cov = _coverage(name, dtype)
            if cov is not None and cov < hidden:
                continue
            _check(_run(X, W, dtype, variant=v), ref, dtype, f"{dtype} hidden={hidden} {name}")
            ran += 1
        assert ran >= 2


@pytest.mark.parametrize("dtype", DTYPES)
def test_rms_norm_general_kernel_odd_rows_and_misaligned(orc, dtype):
    for hidden in (1, 3, 1001):
        X, W = _inputs(dtype, 5, hidden, seed=40 + hidden, small_rows=1)
        assert gm.rms_norm_variant(5, hidden, gm.DTYPE_CODES[dtype]) == 0     # rows not a 16-byte multiple
        _check(_run(X, W, dtype), _ref(orc, X, W, dtype), dtype, f"{dtype} hidden={hidden}")
    # a 2048-wide row whose x and y start one element past 16-byte alignment
    X, W = _inputs(dtype, 9, 2048, seed=50)
    _check(_run(X, W, dtype, offset=1), _ref(orc, X, W, dtype), dtype, f"{dtype} misaligned")


@pytest.mark.parametrize("dtype", DTYPES)
def test_rms_norm_without_weight_in_place_and_eps(orc, dtype):
    X, _ = _inputs(dtype, 12, 2048, seed=60, small_rows=4, weight=False)
    _check(_run(X, None, dtype), _ref(orc, X, None, dtype), dtype, f"{dtype} no weight")
    X, W = _inputs(dtype, 12, 1024, seed=61, small_rows=4)
    _check(_run(X, W, dtype, in_place=True), _ref(orc, X, W, dtype), dtype, f"{dtype} in place")
    for eps in (0.0, 1e-2):
        _check(_run(X, W, dtype, eps=eps), _ref(orc, X, W, dtype, eps=eps), dtype, f"{dtype} eps={eps}")


def test_rms_norm_long_rows(orc):
    """The longest vector row (32768 floats over 16 waves) and one element
    beyond it (the general kernel)."""
    for hidden, expect in ((32768, "vec nv8 w16"), (32772, "general")):
        X, W = _inputs("f32", 3, hidden, seed=hidden)
        assert gm.rms_norm_variant_names()[gm.rms_norm_variant(3, hidden, gm.F32)] == expect
        _check(_run(X, W, "f32"), _ref(orc, X, W, "f32"), "f32", f"hidden={hidden}")


def test_rms_norm_rows_beyond_one_launch(orc):
    """More rows than one launch covers (2^20 workgroups): the call splits
    them over several launches on the stream."""
    rows = (1 << 20) * 4 + 3          # vector variant, 4 rows per workgroup
    X, W = _inputs("f32", rows, 4, seed=70)
    _check(_run(X, W, "f32"), _ref(orc, X, W, "f32"), "f32", "4M+3 rows")
    rows = (1 << 20) + 5              # general kernel, one row per workgroup
    X, W = _inputs("bf16", rows, 3, seed=71)
    _check(_run(X, W, "bf16"), _ref(orc, X, W, "bf16"), "bf16", "1M+5 rows general")


def test_rms_norm_deterministic():
    for dtype, hidden, v in (("bf16", 3584, -1), ("f32", 2048, -1), ("f32", 8192, 16), ("f16", 1001, 0)):
        X, W = _inputs(dtype, 64, hidden, seed=80)
        assert_bits_equal(_run(X, W, dtype, variant=v), _run(X, W, dtype, variant=v), f"{dtype} {hidden}")


@pytest.mark.parametrize("key", sorted(workloads.RMSNORM_WORKLOADS))
def test_rms_norm_workload_parity(orc, key):
    """The workloads bench.py times, in the variant it times: the page's
    32-row example in full, the large ones on 256 sampled rows (rows are
    independent, so the oracle normalises just those)."""
    w = workloads.RMSNORM_WORKLOADS[key]
    X, W = workloads.make_rms_inputs(w)
    Y = _run(X, W, w.dtype, eps=w.eps)
    rows = np.arange(w.rows) if w.rows <= 256 else np.sort(np.random.default_rng(1).choice(w.rows, 256, False))
    ref = orc.rms_norm64(np.ascontiguousarray(X[rows]), W, w.eps, w.dtype)
    _check(Y[rows], ref, w.dtype, key)


def test_rms_norm_empty():
    import torch

    x = torch.empty((0, 64), device="cuda")
    assert gm.rms_norm(x).shape == (0, 64)
    x = torch.empty((5, 0), device="cuda", dtype=torch.bfloat16)
    assert gm.rms_norm(x).shape == (5, 0)


def test_rms_norm_partial_overlap_is_refused():
    """y may be x itself, but an output that starts one row into x (or lies
    over the weight) is refused before any launch, and x is left as it was."""
    import torch

    rows, hidden = 16, 256
    buf = torch.randn(rows * hidden + hidden, device="cuda")
    x = buf[:rows * hidden].view(rows, hidden)
    before = x.clone()
    with pytest.raises(gm.GemmMklError) as e:
        gm.rms_norm(x, out=buf[hidden:].view(rows, hidden))
    assert e.value.status == -1
    w = torch.ones(hidden, device="cuda")
    y = torch.empty(rows, hidden, device="cuda")
    with pytest.raises(gm.GemmMklError) as e:
        gm.rms_norm(x, y[1], out=y)
    assert e.value.status == -1
    torch.cuda.synchronize()
    assert torch.equal(x, before)
    xi = x.clone()
    gm.rms_norm(xi, w, out=xi)   # in place stays allowed
    assert torch.equal(gm.rms_norm(x, w), xi)


@pytest.mark.parametrize("hidden", (256, 301))
@pytest.mark.parametrize("dtype", DTYPES)
def test_rms_norm_special_values(orc, dtype, hidden):
    """Rows holding +inf, -inf or NaN, and an all-zero row, through the vector
    (256) and the general (301) kernel.  A row with an infinity has an
    infinite sum of squares, so its scale is 0: the infinite element becomes
    NaN (inf * 0) and every other element a signed zero, on both sides.  A
    NaN row is all NaN; a zero row stays zero (the scale is 1/sqrt(eps)).
    The special rows must match the oracle's rounding bit for bit (NaN as a
    pattern), the ordinary rows within the tolerance."""
    rng = np.random.default_rng(90)
    x = rng.standard_normal((6, hidden))
    x[1, 5] = np.inf
    x[2, hidden - 1] = -np.inf
    x[3, 7] = np.nan
    x[4, :] = 0.0
    w = 1.0 + 0.5 * rng.standard_normal(hidden)
    X, W = workloads.to_storage(x, dtype), workloads.to_storage(w, dtype)
    Y = _run(X, W, dtype)
    y64 = orc.rms_norm64(X, W, EPS, dtype)
    got = widen_bits(Y, dtype)
    assert np.array_equal(np.isnan(got), np.isnan(y64)), "NaN pattern"
    assert np.isnan(y64[1, 5]) and np.isnan(y64[2, hidden - 1]) and np.isnan(y64[3]).all()
    special = np.array([1, 2, 3, 4])
    ref = orc.round_to_dtype(y64[special], dtype)
    num = ~np.isnan(y64[special])
    assert_bits_equal(Y[special][num], ref[num], f"{dtype} H={hidden} special rows")
    _check(Y[[0, 5]], y64[[0, 5]], dtype, f"{dtype} H={hidden} ordinary rows")
