"""CPU tests of the oracle: every pin must hold, and planted mistakes must be caught.

The oracle is what the GPU path is checked against, so it is pinned to facts
outside itself (see ``oracle_pins.py``).  The second half plants plausible
mistakes into copies of the oracle's C source (on the CPU only) and checks
that at least one pin fails for each of them.
"""
import os
import shutil
import subprocess

import pytest

import oracle
import oracle_pins

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(orc, check):
    check(orc.load())


# (description, text to replace in gemm_oracle.c, replacement, pins expected to catch it)
MUTANTS = [
    ("wrong sign of the products", "acc += widen(A", "acc -= widen(A",
     ["check_closed_form_all_ones"]),
    ("dropped last term of the sum", "for (int64_t k = 0; k < K; ++k)\n        acc +=",
     "for (int64_t k = 0; k + 1 < K; ++k)\n        acc +=", ["check_closed_form_all_ones"]),
    ("B read with A's row count (wrong batch stride)", "(l * N + n) * K, K);",
     "(l * M + n) * K, K);", ["check_bruteforce_fraction"]),
    ("transposed output", "C64[(l * M + m) * N + n] =", "C64[(l * N + n) * M + m] =",
     ["check_bruteforce_fraction"]),
    ("B indexed [K][N] instead of [N][K]", "widen(B, dtype, b_off + k)",
     "widen(B, dtype, (b_off / K) + k)", ["check_bruteforce_fraction"]),
    ("ReLU keeps -0", "return (x > 0.0) ? x : 0.0;", "return (x >= 0.0) ? x : 0.0;",
     ["check_epilogue_values"]),
    ("ReLU passes NaN through", "return (x > 0.0) ? x : 0.0;", "return (x <= 0.0) ? 0.0 : x;",
     ["check_special_values"]),
    ("fp16 infinity encoded as the largest finite value", "if (isinf(a)) return sign | 0x7c00;",
     "if (isinf(a)) return sign | 0x7bff;", ["check_special_values"]),
    ("SiLU with the wrong sign in exp", "return x / (1.0 + exp(-x));",
     "return x / (1.0 + exp(x));", ["check_epilogue_values"]),
    ("fp16 subnormal scale off by one", "ldexp((double)f, -24)", "ldexp((double)f, -25)",
     ["check_widen_f16_exhaustive"]),
    ("ties away from zero instead of to even", "double q = rint(", "double q = round(",
     ["check_round_bf16_midpoints"]),
    ("double rounding through binary32", "encode_bf16(round_to_format(x, 8,",
     "encode_bf16(round_to_format((float)x, 8,", ["check_round_bf16_midpoints"]),
    ("epilogue applied to the products instead of the sum",
     "acc += widen(A, dtype, a_off + k) * widen(B, dtype, b_off + k);",
     "acc += oracle_epilogue(widen(A, dtype, a_off + k) * widen(B, dtype, b_off + k), 1);",
     ["check_bruteforce_fraction"]),
    ("grouped: a row assigned to the next group", "while (g < G && offs[g] <= r)",
     "while (g < G && offs[g] < r)", ["check_grouped_vs_numpy"]),
    ("grouped: B of the wrong group", "dot_row(A, B, dtype, r * K, (g * N + n) * K, K)",
     "dot_row(A, B, dtype, r * K, ((g > 0 ? g - 1 : 0) * N + n) * K, K)", ["check_grouped_vs_numpy"]),
    ("grouped: rows in no group written", "        if (g == G)\n            continue;\n",
     "        if (g == G)\n            g = G - 1;\n", ["check_grouped_vs_numpy"]),
    ("RMSNorm: mean over H - 1 entries", "sqrt(ss / (double)H + eps)", "sqrt(ss / (double)(H - 1) + eps)",
     ["check_rms_norm_vs_torch_and_mp", "check_rms_norm_invariants"]),
    ("RMSNorm: eps outside the square root", "1.0 / sqrt(ss / (double)H + eps)",
     "1.0 / (sqrt(ss / (double)H) + eps)", ["check_rms_norm_closed_forms"]),
    ("RMSNorm: weight indexed by row", "* widen(w, dtype, j)", "* widen(w, dtype, r)",
     ["check_rms_norm_vs_torch_and_mp", "check_rms_norm_invariants"]),
    ("RMSNorm: first square dropped", "for (int64_t j = 0; j < H; ++j) {\n            double v",
     "for (int64_t j = 1; j < H; ++j) {\n            double v", ["check_rms_norm_vs_torch_and_mp"]),
    ("RMSNorm: rows share the first row's sum", "widen(x, dtype, r * H + j);\n            ss",
     "widen(x, dtype, j);\n            ss", ["check_rms_norm_vs_torch_and_mp", "check_rms_norm_invariants"]),
]


@pytest.mark.parametrize("desc,old,new,catchers", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, desc, old, new, catchers):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(os.path.join(os.path.dirname(oracle.__file__), "gemm_oracle.c")).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new))
    so = str(tmp_path / "libmutant.so")
    try:
        oracle.oracle.compile_source(str(mutant), so)
    except subprocess.CalledProcessError as e:  # pragma: no cover
        pytest.fail(f"mutant does not compile: {e}")
    lib = oracle.load(so)
    by_name = {f.__name__: f for f in oracle_pins.ALL_CHECKS}
    caught = []
    for name in catchers:
        try:
            by_name[name](lib)
        except AssertionError:
            caught.append(name)
    assert caught, f"planted mistake '{desc}' passed every pin in {catchers}"
