"""CPU tests of the C ABI: exported symbols, argument checks, plans.

No call here reaches a kernel launch: every call is either rejected by the
argument checks (which run before any HIP call) or describes an empty problem.
"""
import ctypes
import os
import re

import pytest

import tiled_dense_gemm_mkl_amd as gm
from tiled_dense_gemm_mkl_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_mkl.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gm.LIB_PATH):
        pytest.skip("libgemm_mkl.so is not built (run python -m tiled_dense_gemm_mkl_amd.build)")
    return gm.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(gemm_mkl\w*)\s*\(", text)
    return sorted(set(names))


def test_header_declares_what_the_binding_expects():
    assert declared_functions() == sorted(gm.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} is declared in gemm_mkl.h but not exported"


def test_version(lib):
    assert lib.gemm_mkl_version() >= 100


BF16, F32, F16 = gm.BF16, gm.F32, gm.F16
ID, RELU, SILU = gm.EPI_IDENTITY, gm.EPI_RELU, gm.EPI_SILU
FAKE = 0x10000  # never dereferenced: every call below is rejected before any launch
# distinct fake operands, 1 TiB apart, for checks that come after the one that
# rejects operands sharing bytes
FA, FB, FC, FD = 1 << 40, 2 << 40, 3 << 40, 4 << 40


@pytest.mark.parametrize("args,status", [
    ((FAKE, FAKE, FAKE, 4, 4, 4, 1, 7, ID), -2),            # unknown dtype
    ((FAKE, FAKE, FAKE, 4, 4, 4, 1, -1, ID), -2),
    ((FAKE, FAKE, FAKE, 4, 4, 4, 1, BF16, 3), -3),          # unknown epilogue
    ((FAKE, FAKE, FAKE, -1, 4, 4, 1, BF16, ID), -1),        # negative sizes
    ((FAKE, FAKE, FAKE, 4, -4, 4, 1, BF16, ID), -1),
    ((FAKE, FAKE, FAKE, 4, 4, -4, 1, BF16, ID), -1),
    ((FAKE, FAKE, FAKE, 4, 4, 4, -1, BF16, ID), -1),
    ((FAKE, FAKE, None, 4, 4, 4, 1, BF16, ID), -1),         # null C
    ((None, FAKE, FAKE, 4, 4, 4, 1, BF16, ID), -1),         # null A with K > 0
    ((FAKE, None, FAKE, 4, 4, 4, 1, F32, RELU), -1),        # null B with K > 0
    ((FAKE + 1, FAKE, FAKE, 4, 4, 4, 1, BF16, ID), -1),     # A not aligned to its element
    ((FAKE, FAKE, FAKE + 2, 4, 4, 4, 1, F32, ID), -1),      # C not aligned to fp32
    ((FAKE, FAKE, FAKE, 2 ** 40, 2 ** 40, 2 ** 40, 1, BF16, ID), -1),  # byte sizes overflow
    ((None, None, None, 0, 4, 4, 1, BF16, ID), 0),          # empty problems: no launch
    ((None, None, None, 4, 0, 4, 1, F32, SILU), 0),
    ((None, None, None, 4, 4, 4, 0, F16, RELU), 0),
    ((None, None, None, 0, 0, 0, 0, BF16, ID), 0),
])
def test_argument_checks(lib, args, status):
    assert gm.gemm_mkl(*args, None) == status


def test_dtype_checked_before_epilogue(lib):
    assert gm.gemm_mkl(FAKE, FAKE, FAKE, 4, 4, 4, 1, 9, 9, None) == -2


@pytest.mark.parametrize("kw,status", [
    (dict(prefetch_stages=-2), -1),       # a negative prefetch depth is invalid
    (dict(prefetch_stages=-7), -1),
    (dict(split_k=-1), -1),
    (dict(config_id=-5), -1),
    (dict(config_id=10_000), -6),         # no such configuration
    (dict(prefetch_stages=9), -6),        # no kernel with that ring depth
    (dict(split_k=17), -6),
])
def test_option_checks(lib, kw, status):
    o = gm.make_opts(**kw)
    assert gm.gemm_mkl_ex(FAKE, FAKE, None, 4, 4, 4, 1, BF16, ID, None, o) in (status, -1)
    # the plan query applies the same checks without pointers
    try:
        gm.get_plan(64, 64, 64, 1, BF16, ID, o)
        got = 0
    except gm.GemmMklError as e:
        got = e.status
    assert got == status


def test_config_of_another_dtype_is_not_available(lib):
    names = gm.config_names()
    f32_ids = [i for i, n in enumerate(names) if n.startswith("f32")]
    assert f32_ids
    with pytest.raises(gm.GemmMklError) as e:
        gm.get_plan(256, 256, 256, 1, BF16, ID, gm.make_opts(config_id=f32_ids[0]))
    assert e.value.status == -6


def test_workspace_flags_and_alignment(lib):
    o = gm.make_opts(workspace_ptr=FAKE + 16, workspace_bytes=1 << 20)  # not 256-byte aligned
    with pytest.raises(gm.GemmMklError):
        gm.get_plan(64, 64, 64, 1, BF16, ID, o)
    o = gm.make_opts()
    o.flags = 0x100  # unknown flag bit
    with pytest.raises(gm.GemmMklError):
        gm.get_plan(64, 64, 64, 1, BF16, ID, o)


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, 123):
        s = gm.status_string(code)
        assert isinstance(s, str) and s
    assert "prefetch_stages" in gm.status_string(-1)
    assert gm.status_string(0) == "success"
    assert gm.status_string(123) == "unknown status"


def test_config_table(lib):
    names = gm.config_names()
    assert len(names) == lib.gemm_mkl_num_configs() >= 3
    for prefix in ("f32", "f16", "bf16"):
        assert any(n.startswith(prefix + " ") for n in names)
    assert lib.gemm_mkl_config_name(-1) is None
    assert lib.gemm_mkl_config_name(len(names)) is None


@pytest.mark.parametrize("key", list(workloads.WORKLOADS))
def test_plans_of_the_workloads(lib, key):
    w = workloads.WORKLOADS[key]
    code = gm.DTYPE_CODES[w.dtype]
    epi = gm.EPILOGUE_CODES[w.epilogue]
    p = gm.get_plan(w.M, w.N, w.K, w.L, code, epi)
    assert p["general"] == 0
    tiles = -(-w.M // p["block_m"]) * -(-w.N // p["block_n"]) * w.L
    es = 4 if w.dtype == "f32" else 2
    assert p["block_k"] * es in (64, 128)
    if p["streamk"]:
        chunks = -(-w.K // p["block_k"])
        need = -(-chunks // 7)
        assert p["split_k"] == 1 and p["grid"] == max(1, min(256, tiles * chunks // need))
        assert p["workspace_bytes"] == p["counter_bytes"] + 2 * p["grid"] * p["block_m"] * p["block_n"] * 4
    elif p["fixup"]:
        # split-K summed in the kernel: the pieces of a tile share an XCD
        assert p["grid"] == -(-tiles // 8) * 8 * p["split_k"]
    else:
        assert p["grid"] == tiles * p["split_k"]
    if p["streamk"]:
        pass
    elif p["fixup"]:
        assert p["workspace_bytes"] == p["counter_bytes"] + tiles * p["split_k"] * p["block_m"] * p["block_n"] * 4
    elif p["split_k"] > 1:
        assert p["workspace_bytes"] == p["split_k"] * w.L * w.M * w.N * 4
    else:
        assert p["workspace_bytes"] == 0
    # a forced split with the reduction kernel: [S][L][M][N] fp32 partials
    p2 = gm.get_plan(w.M, w.N, w.K, w.L, code, epi, gm.make_opts(split_k=2, fixup=False))
    assert p2["split_k"] == 2 and p2["fixup"] == 0 and p2["workspace_bytes"] == 2 * w.L * w.M * w.N * 4
    p3 = gm.get_plan(w.M, w.N, w.K, w.L, code, epi, gm.make_opts(split_k=2))
    assert gm.workspace_size(w.M, w.N, w.K, w.L, code, 2) == p3["workspace_bytes"]


def _round256(n):
    return (n + 255) // 256 * 256


def test_unaligned_K_is_repacked(lib):
    """K * element size not a multiple of 16: A and B are copied into rows of
    Kp elements (K rounded up to 16 bytes) in the workspace, and the plan is
    the aligned plan at Kp; the general kernel runs only when forced."""
    M, N, K, L = 33, 17, 13, 2
    p = gm.get_plan(M, N, K, L, BF16, RELU)          # 26-byte rows
    want = gm.get_plan(M, N, 16, L, BF16, RELU)      # the same call at Kp = 16
    assert p["general"] == 0 and p["packed"] == 1 and want["packed"] == 0
    for key in ("config_id", "prefetch_stages", "split_k", "grid", "block_m", "block_n"):
        assert p[key] == want[key], key
    assert p["workspace_bytes"] == _round256(L * M * 16 * 2) + _round256(L * N * 16 * 2)
    # a forced split: partials first, then the two packed operands
    K2, Kp2 = 1001, 1008
    p2 = gm.get_plan(M, N, K2, L, BF16, RELU, gm.make_opts(split_k=2))
    assert p2["split_k"] == 2 and p2["packed"] == 1
    assert p2["workspace_bytes"] == (_round256(2 * L * M * N * 4) + _round256(L * M * Kp2 * 2)
                                     + _round256(L * N * Kp2 * 2))
    assert gm.workspace_size(M, N, K2, L, BF16, 2) == p2["workspace_bytes"]
    # fp32: rows padded to a multiple of 4 elements
    p3 = gm.get_plan(70, 65, 37, 1, F32, RELU)
    assert p3["packed"] == 1 and p3["workspace_bytes"] == _round256(70 * 40 * 4) + _round256(65 * 40 * 4)
    # the general kernel when forced; stream-K and the persistent grid are not
    # offered on repacked operands
    g = gm.get_plan(M, N, K, L, BF16, RELU, gm.make_opts(force_general=True))
    assert g["general"] == 1 and g["packed"] == 0 and g["workspace_bytes"] == 0
    for opts in (gm.make_opts(streamk=True), gm.make_opts(persistent=True)):
        with pytest.raises(gm.GemmMklError) as e:
            gm.get_plan(M, N, K, L, BF16, RELU, opts)
        assert e.value.status == -6
    # aligned K is not repacked
    assert gm.get_plan(M, N, 16, L, BF16, RELU)["packed"] == 0


def test_every_prefetch_depth_of_a_config_is_plannable(lib):
    names = gm.config_names()
    for cid, name in enumerate(names):
        dt = gm.DTYPE_CODES[name.split()[0]]
        ok = []
        for p in range(0, 9):
            try:
                plan = gm.get_plan(300, 300, 1000, 1, dt, ID, gm.make_opts(config_id=cid, prefetch_stages=p))
                assert plan["prefetch_stages"] == p and plan["config_id"] == cid
                ok.append(p)
            except gm.GemmMklError as e:
                assert e.status == -6
        assert ok, f"config {name} has no prefetch depth"


def test_streamk_plans(lib):
    # the headline shape leaves 80 of 256 CUs idle with 128x128 tiles: stream-K
    # spreads its 176 x 32 chunk units evenly
    p = gm.get_plan(512, 5632, 2048, 1, BF16, RELU, gm.make_opts(streamk=True))
    assert p["streamk"] == 1 and p["grid"] == 256 and p["split_k"] == 1
    assert p["counter_bytes"] % 256 == 0 and p["workspace_bytes"] > p["counter_bytes"]
    p = gm.get_plan(512, 5632, 2048, 1, BF16, RELU, gm.make_opts(streamk=False))
    assert p["streamk"] == 0
    o = gm.make_opts()
    o.flags = 2 | 4  # both forced and forbidden
    with pytest.raises(gm.GemmMklError) as e:
        gm.get_plan(64, 64, 64, 1, BF16, ID, o)
    assert e.value.status == -1


def test_ctypes_struct_sizes_match_header(lib):
    # gemm_mkl_opts: 4 x int32, pointer, size_t
    # gemm_mkl_plan: 4 x int32, int64, 4 x int32, size_t, 5 x int32 (+ 4 bytes of tail padding)
    assert ctypes.sizeof(gm._binding.Opts) == 32
    assert ctypes.sizeof(gm._binding.Plan) == 72


def test_streamk_only_where_instantiated(lib):
    # regression: a prefetch depth beyond the launch table once spilled tile
    # launchers into the stream-K table of a configuration; stream-K plans
    # must exist exactly for the configurations built with stream-K kernels
    have = set()
    for cid, name in enumerate(gm.config_names()):
        dt = gm.DTYPE_CODES[name.split()[0]]
        for p in range(0, 9):
            try:
                plan = gm.get_plan(300, 200, 2112, 2, dt, ID, gm.make_opts(config_id=cid, prefetch_stages=p,
                                                                             streamk=True))
            except gm.GemmMklError as e:
                assert e.status == -6
                continue
            assert plan["streamk"] == 1
            have.add((name, p))
    want = {("f32 64x64 k32 waves2x2 mfma32", 2),
            ("f16 128x256 k64 waves2x2 mfma32", 2), ("bf16 128x256 k64 waves2x2 mfma32", 2),
            ("f16 128x128 k64 waves2x2 mfma32", 2), ("f16 128x128 k64 waves2x2 mfma32", 3),
            ("bf16 128x128 k64 waves2x2 mfma32", 2), ("bf16 128x128 k64 waves2x2 mfma32", 3)}
    assert have == want


@pytest.mark.parametrize("args,status", [
    # (A, B, C, offs, G, total_m, N, K, dtype, epilogue)
    ((FAKE, FAKE, FAKE, FAKE, 2, 8, 8, 8, 7, ID), -2),          # unknown dtype
    ((FAKE, FAKE, FAKE, FAKE, 2, 8, 8, 8, BF16, 5), -3),        # unknown epilogue
    ((FAKE, FAKE, FAKE, FAKE, -1, 8, 8, 8, BF16, ID), -1),      # negative sizes
    ((FAKE, FAKE, FAKE, FAKE, 2, -8, 8, 8, BF16, ID), -1),
    ((FAKE, FAKE, FAKE, FAKE, 2, 8, -8, 8, BF16, ID), -1),
    ((FAKE, FAKE, FAKE, FAKE, 2, 8, 8, -8, BF16, ID), -1),
    ((FAKE, FAKE, FAKE, FAKE, 65537, 8, 8, 8, BF16, ID), -1),  # too many groups
    ((FAKE, FAKE, FAKE, FAKE, 2, 2 ** 31, 8, 8, BF16, ID), -1),  # rows beyond int32
    ((FAKE, FAKE, None, FAKE, 2, 8, 8, 8, BF16, ID), -1),       # null C
    ((FAKE, FAKE, FAKE, None, 2, 8, 8, 8, BF16, ID), -1),       # null offsets
    ((None, FAKE, FAKE, FAKE, 2, 8, 8, 8, BF16, ID), -1),       # null A with K > 0
    ((FAKE + 2, FAKE, FAKE, FAKE, 2, 8, 8, 8, F32, ID), -1),    # A not element-aligned
    ((FAKE, FAKE, FAKE, FAKE + 2, 2, 8, 8, 8, BF16, ID), -1),   # offsets not int32-aligned
    ((None, None, None, None, 0, 8, 8, 8, BF16, ID), 0),        # no groups: no launch
    ((None, None, None, None, 2, 0, 8, 8, F16, RELU), 0),       # no rows
    ((None, None, None, None, 2, 8, 0, 8, F32, SILU), 0),       # no columns
])
def test_grouped_argument_checks(lib, args, status):
    assert gm.gemm_mkl_grouped(*args, None, None) == status


def test_grouped_option_checks(lib):
    ok = (None, None, None, None, 0, 8, 8, 8, BF16, ID, None)
    assert gm.gemm_mkl_grouped(*ok, gm.make_opts(split_k=2)) == -6       # groups are never split
    o = gm.make_opts()
    o.flags = 2
    assert gm.gemm_mkl_grouped(*ok, o) == -6                              # no stream-K
    assert gm.gemm_mkl_grouped(*ok, gm.make_opts(prefetch_stages=-3)) == -1
    args = (FA, FB, FC, FD, 2, 8, 8, 64, BF16, ID, None)
    assert gm.gemm_mkl_grouped(*args, gm.make_opts(config_id=10_000)) == -6  # no such configuration
    f32_ids = [i for i, n in enumerate(gm.config_names()) if n.startswith("f32")]
    assert gm.gemm_mkl_grouped(*args, gm.make_opts(config_id=f32_ids[0])) == -6  # another dtype's


def test_grouped_config_query(lib):
    names = gm.config_names()
    # 4096 rows in 8 groups x 5632 x 2048: 256 x 256 tiles with 8 waves (the
    # partly filled last tile of each group skips its empty row blocks)
    cid = gm.grouped_config(8, 4096, 5632, 2048, BF16, RELU)
    assert names[cid] == "bf16 256x256 k64 waves2x4 mfma32"
    # 16 groups of about 64 rows: 128-row tiles
    cid = gm.grouped_config(16, 1024, 4096, 1024, BF16, RELU)
    assert names[cid].startswith("bf16 128x128")
    cid = gm.grouped_config(1, 8192, 8192, 8192, F16, ID)
    assert names[cid].startswith("f16 256x256")
    cid = gm.grouped_config(4, 1000, 300, 256, F32, SILU)
    assert names[cid].startswith("f32")
    # K * 2 bytes not a multiple of 16: planned at the repacked K = 16
    assert gm.grouped_config(4, 100, 64, 9, BF16, ID) == gm.grouped_config(4, 100, 64, 16, BF16, ID)
    with pytest.raises(gm.GemmMklError) as e:
        gm.grouped_config(-1, 100, 64, 64, BF16, ID)
    assert e.value.status == -1
    with pytest.raises(gm.GemmMklError) as e:
        gm.grouped_config(4, 100, 64, 64, 9, ID)
    assert e.value.status == -2


# ------------------------------------------------------------------ RMSNorm

@pytest.mark.parametrize("args,status", [
    # (x, weight, y, rows, hidden, eps, dtype, variant)
    ((FAKE, FAKE, FAKE, 4, 64, 1e-6, 7, -1), -2),                   # unknown dtype
    ((FAKE, FAKE, FAKE, -1, 64, 1e-6, F32, -1), -1),                # negative sizes
    ((FAKE, FAKE, FAKE, 4, -64, 1e-6, F32, -1), -1),
    ((FAKE, FAKE, FAKE, 4, 2 ** 31, 1e-6, BF16, -1), -1),           # hidden beyond int32
    ((FAKE, FAKE, FAKE, 2 ** 62, 2 ** 20, 1e-6, F32, -1), -1),      # size overflow
    ((FAKE, FAKE, FAKE, 4, 64, -1e-6, F32, -1), -1),                # eps < 0
    ((FAKE, FAKE, FAKE, 4, 64, float("nan"), F32, -1), -1),         # eps NaN
    ((FAKE, FAKE, FAKE, 4, 64, float("inf"), F32, -1), -1),         # eps infinite
    ((None, FAKE, FAKE, 4, 64, 1e-6, F32, -1), -1),                 # null x
    ((FAKE, FAKE, None, 4, 64, 1e-6, F32, -1), -1),                 # null y
    ((FAKE + 2, FAKE, FAKE, 4, 64, 1e-6, F32, -1), -1),             # x not element-aligned
    ((FAKE, FAKE + 1, FAKE, 4, 64, 1e-6, BF16, -1), -1),            # weight not element-aligned
    ((FAKE, FAKE, FAKE, 4, 64, 1e-6, F32, 99), -1),                 # no such variant
    ((FAKE, FAKE, FAKE, 4, 64, 1e-6, F32, -2), -1),
    ((FA + 4, FB, FC, 4, 64, 1e-6, F32, 1), -6),              # vector variant, x not 16-byte aligned
    ((FA, FB, FC, 4, 3, 1e-6, F32, 1), -6),                   # vector variant, row not 16-byte multiple
    ((FA, FB, FC, 4, 512, 1e-6, F32, 1), -6),                 # vector variant covering 256 floats
    ((None, None, None, 0, 64, 1e-6, F32, -1), 0),                  # no rows: no launch
    ((None, None, None, 4, 0, 1e-6, BF16, -1), 0),                  # no columns
])
def test_rms_norm_argument_checks(lib, args, status):
    x, w, y, rows, hidden, eps, dtype, variant = args
    assert gm.gemm_mkl_rms_norm(x, w, y, rows, hidden, eps, dtype, None, variant) == status


def test_rms_norm_plain_entry_matches_ex_checks(lib):
    assert lib.gemm_mkl_rms_norm(None, None, None, 0, 8, 1e-6, F32, None) == 0
    assert lib.gemm_mkl_rms_norm(FAKE, FAKE, FAKE, 4, 64, -1.0, F32, None) == -1
    assert lib.gemm_mkl_rms_norm(FAKE, FAKE, FAKE, 4, 64, 1e-6, 3, None) == -2


def test_rms_norm_variant_choice(lib):
    names = gm.rms_norm_variant_names()
    assert names[0] == "general" and len(names) == lib.gemm_mkl_rms_norm_num_variants()
    assert lib.gemm_mkl_rms_norm_variant_name(len(names)) is None
    pick = lambda rows, h, dt, al=True: names[gm.rms_norm_variant(rows, h, dt, al)]
    assert pick(32, 2048, F32) == "vec nv1 w8"          # one vector of 4 floats per lane, 8 waves
    assert pick(32, 2048, BF16) == "vec nv4 w1"
    assert pick(32, 3584, BF16) == "vec nv1 w8"         # a partly filled last vector step
    assert pick(32, 8192, BF16) == "vec nv4 w4"
    assert pick(32, 256, F16) == "vec nv1 w1"
    assert pick(4, 32768, F32) == "vec nv8 w16"         # the longest vector row
    assert pick(4, 32772, F32) == "general"             # beyond every vector variant
    assert pick(4, 3, F32) == "general"                 # 12-byte rows
    assert pick(4, 2048, F32, False) == "general"       # unaligned pointers
    with pytest.raises(gm.GemmMklError):
        gm.rms_norm_variant(4, 64, 9)


# ------------------------------------------------------------------ persistent grid

def test_persistent_plans(lib):
    names = gm.config_names()
    cid = names.index("bf16 128x128 k64 waves2x2+4p mfma32")
    # opt-in: the automatic plan keeps the data-parallel grid
    p = gm.get_plan(4096, 5632, 2048, 1, BF16, RELU, gm.make_opts(config_id=cid))
    assert p["persistent"] == 0 and p["grid"] == 1408
    # forced with more tiles than compute units: one workgroup per CU
    p = gm.get_plan(4096, 5632, 2048, 1, BF16, RELU, gm.make_opts(config_id=cid, persistent=True))
    assert p["persistent"] == 1 and p["grid"] == 256 and p["split_k"] == 1 and p["prefetch_stages"] == 3
    # forced on a small problem: one workgroup per tile
    p = gm.get_plan(300, 200, 2112, 2, BF16, SILU, gm.make_opts(config_id=cid, persistent=True))
    assert p["persistent"] == 1 and p["grid"] == 3 * 2 * 2
    # forbidden, or with another depth or a split: not persistent
    assert gm.get_plan(4096, 5632, 2048, 1, BF16, RELU, gm.make_opts(config_id=cid, persistent=False))["persistent"] == 0
    assert gm.get_plan(4096, 5632, 2048, 1, BF16, RELU, gm.make_opts(config_id=cid, prefetch_stages=4))["persistent"] == 0
    assert gm.get_plan(4096, 5632, 2048, 1, BF16, RELU, gm.make_opts(config_id=cid, split_k=2))["persistent"] == 0


def test_persistent_forced_where_unavailable(lib):
    names = gm.config_names()
    f32 = [i for i, n in enumerate(names) if n.startswith("f32")][0]
    for o in (gm.make_opts(config_id=f32, persistent=True),
              gm.make_opts(config_id=names.index("bf16 128x128 k64 waves2x2+4p mfma32"), persistent=True,
                           prefetch_stages=4),
              gm.make_opts(config_id=names.index("bf16 128x128 k64 waves2x2+4p mfma32"), persistent=True,
                           split_k=2)):
        dt = F32 if o.config_id == f32 else BF16
        with pytest.raises(gm.GemmMklError) as e:
            gm.get_plan(1024, 1024, 512, 1, dt, ID, o)
        assert e.value.status == -6
    o = gm.make_opts(persistent=True)
    o.flags |= 16   # with GEMM_MKL_OPT_NO_PERSISTENT
    with pytest.raises(gm.GemmMklError) as e:
        gm.get_plan(1024, 1024, 512, 1, BF16, ID, o)
    assert e.value.status == -1


def test_planning_from_many_threads_matches_serial_planning():
    """The plan cache is shared by all threads: plans made by 8 threads at
    once (cache misses and hits interleaved) equal the plans a fresh process
    makes one by one."""
    import json
    import subprocess
    import sys
    import threading

    shapes = [(m, n, k, l, dt) for m in (1, 97, 513, 1001) for n in (65, 2049, 5633) for k in (8, 528, 2056)
              for l in (1, 3) for dt in (gm.F32, gm.F16, gm.BF16)]
    got, errors = {}, []

    def worker(part):
        try:
            for s in part:
                got[s] = gm.get_plan(*s, gm.EPI_RELU)
        except Exception as e:
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(shapes[i::8] + shapes[(i + 1) % 8::8],)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors
    code = ("import json, sys; import tiled_dense_gemm_mkl_amd as gm; "
            "shapes = json.loads(sys.stdin.read()); "
            "print(json.dumps([gm.get_plan(*s, gm.EPI_RELU) for s in shapes]))")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], input=json.dumps(shapes), capture_output=True, text=True,
                       cwd=root, timeout=120, check=True)
    serial = json.loads(r.stdout)
    assert [got[s] for s in shapes] == serial


def test_noalloc_argument_checks(lib):
    """gemm_mkl_noalloc's checks run before any HIP call: these calls never
    reach the scratch or a kernel."""
    call = lambda M, N, K, L, dtype, epi, o: lib.gemm_mkl_noalloc(  # noqa: E731
        FA, FB, FC, M, N, K, L, dtype, epi, None, ctypes.byref(o) if o is not None else None)
    # a caller workspace makes no sense here
    assert call(64, 64, 64, 1, BF16, ID, gm.make_opts(workspace_ptr=FAKE, workspace_bytes=1 << 20)) == -1
    # the checks of gemm_mkl_ex, in its order
    assert call(64, 64, 64, 1, 7, ID, None) == -2
    assert call(64, 64, 64, 1, BF16, 9, None) == -3
    assert call(-1, 64, 64, 1, BF16, ID, None) == -1
    assert call(64, 64, 64, 1, BF16, ID, gm.make_opts(prefetch_stages=-2)) == -1
    # stream-K is not offered (its counters would have to start at zero)
    assert call(512, 640, 2048, 1, BF16, ID, gm.make_opts(streamk=True)) == -6
    # empty problems launch nothing
    assert call(0, 64, 64, 1, BF16, ID, None) == 0
    # a forced split whose partial sums exceed the scratch
    need = gm.get_plan(512, 4096, 2048, 1, BF16, ID, gm.make_opts(split_k=16))["workspace_bytes"]
    assert need > gm.NOALLOC_SCRATCH_BYTES
    assert call(512, 4096, 2048, 1, BF16, ID, gm.make_opts(split_k=16)) == -4
    # repacked operands that exceed it (K = 2047 bf16: A and B copied, 2 * 4096 * 2048 * 2 B each)
    assert call(4096, 4096, 2047, 2, BF16, ID, None) == -4


def test_library_shares_torchs_hip_runtime():
    # regression: the library loaded before torch bound the system HIP runtime
    # while torch brought its own, and GPU calls then found no device; load()
    # imports torch first so that one runtime serves both
    import subprocess
    import sys

    code = ("import os, tiled_dense_gemm_mkl_amd as gm; gm.config_names(); import torch; "
            "maps = open('/proc/self/maps').read(); "
            "print(len({l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}))")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=root, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip().splitlines()[-1] == "1"


def test_workspace_tensor_must_be_on_the_operands_gpu():
    # regression: gemm() passed any workspace tensor's address to the kernels,
    # so one in host memory would have been written by the GPU at a host address
    import torch

    gpu = torch.device("cuda", 0)
    assert gm._binding._workspace_args(None, gpu) == (None, 0)
    with pytest.raises(ValueError, match="workspace"):
        gm._binding._workspace_args(torch.zeros(64), gpu)
    with pytest.raises(ValueError, match="workspace"):
        gm._binding._workspace_args(torch.zeros(8, 8).t(), torch.device("cpu"))
    with pytest.raises(TypeError, match="workspace"):
        gm._binding._workspace_args(bytearray(64), gpu)
    ptr, nbytes = gm._binding._workspace_args(torch.zeros(64, dtype=torch.float64), torch.device("cpu"))
    assert nbytes == 512 and ptr != 0


def test_operands_that_share_bytes_are_rejected(lib):
    """C is written while A and B are read, so no byte may belong to both; the
    same holds for a caller workspace, the grouped offsets and the RMSNorm's
    x (unless y is x itself) and weight.  Every call here is rejected before
    any HIP call; calls on adjacent, disjoint ranges run in the GPU tests."""
    M, N, K, L = 64, 48, 32, 2
    a_bytes, b_bytes, c_bytes = L * M * K * 2, L * N * K * 2, L * M * N * 2
    ex = lambda A, B, C, opts=None: gm.gemm_mkl_ex(A, B, C, M, N, K, L, BF16, ID, None, opts)  # noqa: E731
    assert ex(FA, FB, FA) == -1                                   # C is A
    assert ex(FA, FB, FB + b_bytes - 2) == -1                     # C starts on B's last element
    assert ex(FA, FB, FA - c_bytes + 2) == -1                     # C ends on A's first element
    assert ex(FA, FB, FB - 2) == -1                               # C straddles B's start
    ws = lambda p, n: gm.make_opts(workspace_ptr=p, workspace_bytes=n)  # noqa: E731
    assert ex(FA, FB, FC, ws(FA + a_bytes - 256, 512)) == -1      # workspace over the end of A
    assert ex(FA, FB, FC, ws(FC - 256, 512)) == -1                # workspace ending inside C
    assert ex(FA, FB, FC, ws(FB - (1 << 20), (1 << 20) + 256)) == -1  # workspace running into B
    # the raw entry point and the no-allocation one check the same
    assert gm.gemm_mkl(FA, FB, FB, M, N, K, L, BF16, ID, None) == -1
    assert lib.gemm_mkl_noalloc(FA, FB, FA + 64, M, N, K, L, BF16, ID, None, None) == -1
    # grouped: C against A, B, offsets; the workspace against all four
    G, T = 3, 40
    g = lambda A, B, C, offs, opts=None: gm.gemm_mkl_grouped(A, B, C, offs, G, T, N, K, BF16, ID, None, opts)  # noqa: E731
    assert g(FA, FB, FA + 2, FD) == -1
    assert g(FA, FB, FB, FD) == -1
    assert g(FA, FB, FC, FC + T * N * 2 - 4) == -1                # offsets on C's last bytes
    assert g(FA, FB, FC, FD, ws(FD - 256, 512)) == -1             # workspace over the offsets
    assert g(FA, FB, FC, FD, ws(FC + 256, 256)) == -1             # workspace inside C
    # RMSNorm: y partly over x, or over the weight
    rows, H = 8, 64
    rms = lambda x, w, y: gm.gemm_mkl_rms_norm(x, w, y, rows, H, 1e-6, F32, None)  # noqa: E731
    assert rms(FA, FB, FA + 4 * H) == -1                          # y one row past x: rows overlap
    assert rms(FA + 4, FB, FA) == -1
    assert rms(FA, FC + 4 * H, FC) == -1                          # the weight inside y
