"""Planted mistakes in copies of the CPU oracle must each fail some pin.

Each mutant replaces one fragment of oracle/zq_ref.c (a dropped term, a wrong
sign, rounding mode, index or operand), builds the copy with gcc into a
temporary directory, routes the oracle wrapper through it and runs every
pin from test_oracle_pins.py.  The test passes when at least one pin fails.
Everything here runs on the CPU.
"""
from __future__ import annotations

import os
import subprocess

import pytest

from oracle import build as obuild
from oracle import ref
from tests import test_oracle_pins as pins

MUTANTS = {
    "round_half_away": ("float r = nearbyintf(t);", "float r = roundf(t);"),
    "scale_over_128": ("float s = a / 127.0f;\n    for (int64_t i = 0;", "float s = a / 128.0f;\n    for (int64_t i = 0;"),
    "unbiased_variance": ("double var = ss / (double)K;", "double var = ss / (double)(K - 1);"),
    "eps_dropped": ("double r = 1.0 / sqrt(var + (double)eps);", "double r = 1.0 / sqrt(var);"),
    "beta_sign": ("* r * g + b);", "* r * g - b);"),
    "gelu_wrong_scale": ("return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));",
                         "return 0.5 * x * (1.0 + erf(x / 2.0));"),
    "gemm_transposed_w": ("(int64_t)Wq[n * K + k]", "(int64_t)Wq[k * N + n]"),
    "group_index_modulo": ("(double)s_w[n / G] * (double)acc[m * N + n];\n            if (bias)",
                           "(double)s_w[n % (N / G)] * (double)acc[m * N + n];\n            if (bias)"),
    "bias_dropped": ("(double)acc[m * N + n];\n            if (bias)\n                v += (double)bias[n];",
                     "(double)acc[m * N + n];\n            if (bias)\n                v += 0.0;"),
    "fp16_truncates": ("double q = nearbyint(ldexp(a, 10 - e));", "double q = floor(ldexp(a, 10 - e));"),
    "outlier_test_inclusive": ("hit = fabsf(Y[m * K + j]) > alpha;", "hit = fabsf(Y[m * K + j]) >= alpha;"),
    "outlier_test_signed": ("hit = fabsf(Y[m * K + j]) > alpha;", "hit = Y[m * K + j] > alpha;"),
    "outlier_absmax_counted": ("if (!in_o[j] && fabsf(y[j]) > a)", "if (fabsf(y[j]) > a)"),
    "outlier_term_dropped": ("                v += a * w;\n", "                v += 0.0 * a * w;\n"),
    "outlier_weight_unrounded": ("double w = (double)zqref_f16_to_f32(zqref_f64_to_f16((double)W[n * K + j]));",
                                 "double w = (double)W[n * K + j];"),
    "outlier_weight_transposed": ("zqref_f64_to_f16((double)W[n * K + j])", "zqref_f64_to_f16((double)W[j * N + n])"),
    "outlier_act_unrounded": ("double a = (double)zqref_f16_to_f32(zqref_f64_to_f16((double)Y[m * K + j]));",
                              "double a = (double)Y[m * K + j];"),
    "ln_mean_not_subtracted": ("Y[row + k] = (float)((load_x(X, x_is_f16, row + k) - mu) * r * g + b);",
                               "Y[row + k] = (float)(load_x(X, x_is_f16, row + k) * r * g + b);"),
    "gelu_before_bias": ("(double)acc[m * N + n];\n            if (bias)\n                v += (double)bias[n];\n"
                         "            if (act == ACT_GELU)\n                v = gelu64(v);",
                         "(double)acc[m * N + n];\n            if (act == ACT_GELU)\n                v = gelu64(v);\n"
                         "            if (bias)\n                v += (double)bias[n];"),
    "gamma_fold_multiplies": ("gamma_out[j] = (float)(g / (double)s[j]);", "gamma_out[j] = (float)(g * (double)s[j]);"),
    "f16_decode_exponent": ("ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)"),
    "f16_decode_subnormal": ("v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    # FP8 (E4M3) variant
    "e4m3_truncates": ("double q = nearbyint(ldexp(a, 3 - e));", "double q = floor(ldexp(a, 3 - e));"),
    "e4m3_subnormals_flushed": ("const double q = nearbyint(ldexp(a, 9));", "const double q = 0.0;"),
    "e4m3_no_nan_code": ("    if (e == 15 && f == 7)\n        return NAN;", "    (void)0;"),
    "e4m3_exponent_bias_8": ("ldexp((double)(8 + f), e - 10)", "ldexp((double)(8 + f), e - 11)"),
    "e4m3_saturates_early": ("if (a >= 448.0)", "if (a >= 240.0)"),
    "fp8_scale_for_240": ("    while (448.0 * ldexp(1.0, e) < (double)a)\n        e++;\n    while (448.0 * ldexp(1.0, e - 1) >= (double)a)",
                          "    while (240.0 * ldexp(1.0, e) < (double)a)\n        e++;\n    while (240.0 * ldexp(1.0, e - 1) >= (double)a)"),
    "fp8_gemm_transposed_w": ("lut[Wq[n * K + k]]", "lut[Wq[k * N + n]]"),
    "smooth_inverted": ("(float)sqrt(a / w)", "(float)sqrt(w / a)"),
    "fold_weight_divides": ("(double)W[n * K + j] * (double)s[j]", "(double)W[n * K + j] / (double)s[j]"),
    # row-subset and unquantized forms, FP8 weight groups
    "linear_rows_gather_slip": ("memcpy(Xs + esz * (size_t)(r * K), (const char *)X + esz * (size_t)(rows[r] * K), esz * (size_t)K);\n    int rc = zqref_prologue(",
                                "memcpy(Xs + esz * (size_t)(r * K), (const char *)X + esz * (size_t)(r * K), esz * (size_t)K);\n    int rc = zqref_prologue("),
    "fp8_group_stride": ("s[g] = pow2_quantize(W + g * G * K, G * K, q + g * G * K);",
                         "s[g] = pow2_quantize(W + g * K, G * K, q + g * G * K);"),
    "float_layer_bias_dropped": ("                if (bias)\n                    v += (double)bias[n];\n                if (act == ACT_GELU)\n                    v = gelu64(v);\n                Y_out[r * N + n] = v;",
                                 "                if (act == ACT_GELU)\n                    v = gelu64(v);\n                Y_out[r * N + n] = v;"),
    "float_layer_transposed_w": ("v += (double)Y[r * K + k] * (double)W[n * K + k];",
                                 "v += (double)Y[r * K + k] * (double)W[k * N + n];"),
    "group_absmax_first_row": ("s_w[g] = absmax_quantize(W + g * G * K, G * K, Wq + g * G * K);",
                               "{ s_w[g] = absmax_quantize(W + g * G * K, K, Wq + g * G * K);\n"
                               "        for (int64_t i = K; i < G * K; i++) {\n"
                               "            float t = nearbyintf(W[g * G * K + i] / s_w[g]);\n"
                               "            Wq[g * G * K + i] = (int8_t)(t > 127 ? 127 : t < -127 ? -127 : t);\n"
                               "        } }"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(obuild.SRC, encoding="utf-8").read()
    assert src.count(old) == 1, f"mutant {name}: fragment not found exactly once"
    mpath = tmp_path / f"{name}.c"
    mpath.write_text(src.replace(old, new), encoding="utf-8")
    lib = tmp_path / f"lib_{name}.so"
    subprocess.run(["gcc", *obuild.CFLAGS, str(mpath), "-o", str(lib), "-lm"], check=True,
                   capture_output=True)
    return str(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    lib = _build_mutant(tmp_path, name, old, new)
    caught = []
    with ref.using_library(lib):
        for pin in pins.ALL_PINS:
            try:
                pin()
            except (AssertionError, ref.OracleError):
                caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"


def test_pins_pass_on_unmodified_copy(tmp_path):
    """The same machinery on an unmodified copy catches nothing."""
    lib = _build_mutant(tmp_path, "identity", "#include <math.h>", "#include <math.h>")
    with ref.using_library(lib):
        for pin in pins.ALL_PINS:
            pin()
