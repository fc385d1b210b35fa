"""Planted mistakes in the oracle must fail at least one pin.

Each case copies oracle.c, applies one textual change (a dropped term, a
wrong sign or index, a transposed operand, a wrong decode constant, a
broken error ratio), builds the copy with gcc and runs all pins against it
in a child process.  The anchors are checked first, so a refactor of
oracle.c that removes one fails loudly instead of silently passing."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "drop_last_k": ("for (int64_t k = 0; k < jb->K; ++k)",
                    "for (int64_t k = 0; k < jb->K - 1; ++k)"),
    "skip_first_k": ("for (int64_t k = 0; k < jb->K; ++k)",
                     "for (int64_t k = 1; k < jb->K; ++k)"),
    "wrong_sign": ("acc[j] += a * b;", "acc[j] -= a * b;"),
    "transposed_b": ("const double b = load_elem(jb->B, jb->dtype, brow + j);",
                     "const double b = load_elem(jb->B, jb->dtype, j * jb->ldb + k);"),
    "transposed_a": ("load_elem(jb->A, jb->dtype, i * jb->lda + k)",
                     "load_elem(jb->A, jb->dtype, k * jb->lda + i)"),
    "b_uses_lda": ("const int64_t brow = k * jb->ldb;",
                   "const int64_t brow = k * jb->lda;"),
    "a_ignores_lda": ("load_elem(jb->A, jb->dtype, i * jb->lda + k)",
                      "load_elem(jb->A, jb->dtype, i * jb->K + k)"),
    "den_signed": ("den[j] += abs_a * fabs(b);", "den[j] += a * b;"),
    "f16_bias": ("mag = ldexp((double)(0x400 | frac), expo - 25);",
                 "mag = ldexp((double)(0x400 | frac), expo - 24);"),
    "f16_no_hidden_bit": ("mag = ldexp((double)(0x400 | frac), expo - 25);",
                          "mag = ldexp((double)frac, expo - 25);"),
    "f16_subnormal": ("mag = ldexp((double)frac, -24);",
                      "mag = ldexp((double)frac, -25);"),
    "f16_sign": ("return sign ? -mag : mag;", "return mag;"),
    "bf16_bias": ("mag = ldexp((double)(0x80 | frac), expo - 134);",
                  "mag = ldexp((double)(0x80 | frac), expo - 133);"),
    "bf16_no_hidden_bit": ("mag = ldexp((double)(0x80 | frac), expo - 134);",
                           "mag = ldexp((double)frac, expo - 134);"),
    "bf16_subnormal": ("mag = ldexp((double)frac, -133);", "mag = ldexp((double)frac, -126);"),
    "bf16_fraction_width": ("const int expo = (h >> 7) & 0xff;\n    const int frac = h & 0x7f;",
                            "const int expo = (h >> 8) & 0x7f;\n    const int frac = h & 0xff;"),
    "bf16_decoded_as_f16": ("    if (dtype == ORACLE_BF16)\n        return oracle_bf16_to_f64",
                            "    if (0)\n        return oracle_bf16_to_f64"),
    "e4m3_bias": ("mag = ldexp((double)(0x8 | frac), expo - 10);",
                  "mag = ldexp((double)(0x8 | frac), expo - 11);"),
    "e4m3_no_hidden_bit": ("mag = ldexp((double)(0x8 | frac), expo - 10);",
                           "mag = ldexp((double)frac, expo - 10);"),
    "e4m3_subnormal": ("mag = ldexp((double)frac, -9);", "mag = ldexp((double)frac, -10);"),
    "e4m3_all_top_exponent_nan": ("if (expo == 0xf && frac == 0x7)", "if (expo == 0xf)"),
    "e4m3_decoded_as_f16": ("    if (dtype == ORACLE_E4M3)\n        return oracle_e4m3_to_f64",
                            "    if (0)\n        return oracle_e4m3_to_f64"),
    "e5m2_bias": ("mag = ldexp((double)(0x4 | frac), expo - 17);",
                  "mag = ldexp((double)(0x4 | frac), expo - 16);"),
    "e5m2_no_hidden_bit": ("mag = ldexp((double)(0x4 | frac), expo - 17);",
                           "mag = ldexp((double)frac, expo - 17);"),
    "e5m2_subnormal": ("mag = ldexp((double)frac, -16);", "mag = ldexp((double)frac, -17);"),
    "e5m2_fraction_width": ("const int expo = (b >> 2) & 0x1f;\n    const int frac = b & 0x3;",
                            "const int expo = (b >> 3) & 0xf;\n    const int frac = b & 0x7;"),
    "e5m2_infinity_as_nan": ("    if (expo == 0x1f)\n        mag = frac ? NAN : INFINITY;",
                             "    if (expo == 0x1f)\n        mag = NAN;"),
    "e5m2_decoded_as_e4m3": ("    if (dtype == ORACLE_E5M2)\n        return oracle_e5m2_to_f64",
                             "    if (dtype == ORACLE_E5M2)\n        return oracle_e4m3_to_f64"),
    "q8_ties_up": ("r = (fmod(f, 2.0) == 0.0) ? f : f + 1.0;", "r = f + 1.0;"),
    "q8_truncate": ("    else if (frac < 0.5)\n        r = f;", "    else if (frac < 0.999)\n        r = f;"),
    "q8_no_low_saturation": ("    if (v <= -128.0)\n        return -128;", "    if (v <= -129.0)\n        return -129;"),
    "q8_high_saturation_off_by_one": ("    if (v >= 127.0)\n        return 127;", "    if (v >= 127.0)\n        return 126;"),
    "trans_a_ignored": ("load_elem(A, dtype, trans_a ? k * lda + i : i * lda + k)",
                        "load_elem(A, dtype, i * lda + k)"),
    "trans_a_swapped_index": ("load_elem(A, dtype, trans_a ? k * lda + i : i * lda + k)",
                              "load_elem(A, dtype, trans_a ? i * lda + k : k * lda + i)"),
    "trans_b_wrong_ld": ("load_elem(B, dtype, trans_b ? j * ldb + k : k * ldb + j)",
                         "load_elem(B, dtype, trans_b ? j * K + k : k * ldb + j)"),
    "entries_drop_k": ("for (int64_t k = 0; k < K; ++k) {",
                       "for (int64_t k = 0; k + 1 < K; ++k) {"),
    "metric_absolute": ("r = diff / den;", "r = diff;"),
    "metric_zero_den_hidden": ("r = (diff == 0.0) ? 0.0 : INFINITY;", "r = 0.0;"),
    "metric_nan_ignored": ("++n_nonfinite;\n                r = INFINITY;",
                           "r = 0.0;"),
    "bt_index_swapped": ("const double bt = load_elem(jb->B, jb->dtype, j * jb->ldb + k);",
                         "const double bt = load_elem(jb->B, jb->dtype, k * jb->ldb + j);"),
    "bt_ignores_ld": ("const double bt = load_elem(jb->B, jb->dtype, j * jb->ldb + k);",
                      "const double bt = load_elem(jb->B, jb->dtype, j * jb->K + k);"),
    "bt_drops_last_k": ("        for (int64_t k = 0; k < jb->K; ++k) {\n            const double a = load_elem(jb->A, jb->dtype, i * jb->lda + k);\n            for (int64_t j = 0; j < jb->N; ++j) {\n                const double bt",
                        "        for (int64_t k = 0; k + 1 < jb->K; ++k) {\n            const double a = load_elem(jb->A, jb->dtype, i * jb->lda + k);\n            for (int64_t j = 0; j < jb->N; ++j) {\n                const double bt"),
    "epi_drop_beta": ("                v += c0;\n", "\n"),
    "epi_bias_by_row": ("v += (double)bias[j];", "v += (double)bias[i % N];"),
    "epi_c0_by_slot": ("load_elem(C0, dtype, i * ldc0 + j)", "load_elem(C0, dtype, t * ldc0 + j)"),
    "epi_relu_wrong_way": ("if (act == 1 && v < 0.0)", "if (act == 1 && v > 0.0)"),
    "epi_scale_no_alpha": ("double d = fabs(alpha) * D[t * ldd + j];", "double d = D[t * ldd + j];"),
    "epi_reads_c0_when_beta_zero": ("if (beta != 0.0) {\n                const double c0",
                                    "if (1) {\n                const double c0"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert old in text, f"anchor for {name} not found in oracle.c"
    src = tmp_path / "oracle_mutant.c"
    src.write_text(text.replace(old, new))
    lib = str(tmp_path / "liboracle_mutant.so")
    oracle.build(str(src), lib)
    res = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "_pin_runner.py"), lib],
                         capture_output=True, text=True, timeout=600)
    assert res.returncode != 0, f"mutant {name} passed every pin:\n{res.stdout}"


def test_unmutated_copy_passes(tmp_path):
    src = tmp_path / "oracle_copy.c"
    src.write_text(open(SRC).read())
    lib = str(tmp_path / "liboracle_copy.so")
    oracle.build(str(src), lib)
    res = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "_pin_runner.py"), lib],
                         capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr


# Planted mistakes in the Python side of the oracle (the INT8 code bounds
# for random-input results), each applied to a copy of oracle/__init__.py
# that is loaded as a separate module over the same, unmutated C library.
PY_SRC = os.path.join(ROOT, "oracle", "__init__.py")
PY_MUTANTS = {
    "q8_bounds_swapped": ("    return _code_of_exact_sum(v, -err, lib=lib), _code_of_exact_sum(v, err, lib=lib)",
                          "    return _code_of_exact_sum(v, err, lib=lib), _code_of_exact_sum(v, -err, lib=lib)"),
    "q8_lo_plus_one": ("    return _code_of_exact_sum(v, -err, lib=lib), ",
                       "    return _code_of_exact_sum(v, -err, lib=lib) + np.int8(1), "),
    "q8_hi_minus_one": (", _code_of_exact_sum(v, err, lib=lib)\n",
                        ", _code_of_exact_sum(v, err, lib=lib) - np.int8(1)\n"),
    "q8_err_doubled": ("    err = np.asarray(err, dtype=np.float64)\n    return _code",
                       "    err = 2.0 * np.asarray(err, dtype=np.float64)\n    return _code"),
    "q8_err_ignored": (", _code_of_exact_sum(v, err, lib=lib)\n",
                       ", _code_of_exact_sum(v, 0.0 * err, lib=lib)\n"),
    "q8_binary64_ends": ("    tie = (s - fl) == 0.5\n", "    tie = np.zeros(np.shape(s), dtype=bool)\n"),
    "q8_tie_side_swapped": ("np.where(tie & (t > 0), fl + 1, np.where(tie & (t < 0), fl, q))",
                            "np.where(tie & (t < 0), fl + 1, np.where(tie & (t > 0), fl, q))"),
    "q8_no_saturation": ("    return np.clip(q, -128, 127).astype(np.int8)",
                         "    return q.astype(np.int8)"),
}


def _mutant_module(text: str):
    import types
    mod = types.ModuleType("oracle_py_mutant")
    mod.__file__ = PY_SRC  # the same directory, so the same liboracle.so
    exec(compile(text, PY_SRC, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_planted_python_mistake_is_caught(name, monkeypatch):
    from tests import oracle_pins
    old, new = PY_MUTANTS[name]
    text = open(PY_SRC).read()
    assert text.count(old) == 1, f"anchor for {name} not found once in oracle/__init__.py"
    monkeypatch.setattr(oracle_pins, "oracle", _mutant_module(text.replace(old, new)))
    with pytest.raises(AssertionError):
        oracle_pins.pin_q8_allowed(oracle.load())


def test_unmutated_python_copy_passes(monkeypatch):
    from tests import oracle_pins
    monkeypatch.setattr(oracle_pins, "oracle", _mutant_module(open(PY_SRC).read()))
    oracle_pins.pin_q8_allowed(oracle.load())
