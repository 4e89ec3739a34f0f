"""Plant plausible mistakes in a copy of the oracle and check that the pins
catch every one of them (mutation testing, CPU only).

Each mutant is the oracle source with one textual substitution, compiled with
gcc into a temporary directory.  The real oracle source is never modified.
"""
import os
import subprocess

import pytest

import oracle
import pins

MUTANTS = {
    "nibble_order_swapped": ("(k % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4)",
                             "(k % 2 == 0) ? (byte >> 4) : (byte & 0x0Fu)", 1),
    "scale_block_32": ("scales_row[k / 16]", "scales_row[k / 32]", 1),
    "scale_block_off_by_one": ("scales_row[k / 16]", "scales_row[(k + 1) / 16 < K / 16 ? (k + 1) / 16 : k / 16]", 1),
    "e4m3_fnuz_bias": ("(int)e - 7);", "(int)e - 8);", 1),
    "e4m3_subnormal_scale": ("ldexp((double)m, -9)", "ldexp((double)m, -10)", 1),
    "e4m3_subnormal_as_normal": ("mag = ldexp((double)m, -9);", "mag = ldexp(1.0 + (double)m / 8.0, -6);", 1),
    "e4m3_nan_dropped": ("if (e == 15 && m == 7)", "if (0)", 1),
    "e4m3_mantissa_width": ("(double)m / 8.0", "(double)m / 16.0", 1),
    "e2m1_subnormal": ("mag = 0.5 * (double)m;", "mag = 1.0 * (double)m;", 1),
    "e2m1_bias": ("(int)e - 1);", "(int)e);", 1),
    "e2m1_sign_dropped": ("return sign ? -mag : mag;", "return mag;", 1),
    "e4m3_sign_dropped": ("return sign ? -mag : mag;\n}\n\n/* bf16", "return mag;\n}\n\n/* bf16", 1),
    "global_scale_dropped": ("* s * g;", "* s;", 1),
    "global_scale_divides": ("* s * g;", "* s / g;", 1),
    "codes_row_stride": ("j->codes + n * (j->K / 2)", "j->codes + n * (j->K / 4)", 1),
    "scales_row_stride": ("j->scales + n * (j->K / 16)", "j->scales + n * (j->K / 32)", 1),
    "x_transposed": ("const double *xm = xd + m * j->K;", "const double *xm = xd + m;", 1),
    "abs_dropped": ("absacc += fabs(t);", "absacc += t;", 1),
    "last_k_dropped": ("for (int64_t k = 0; k < j->K; ++k) {\n                double t",
                       "for (int64_t k = 0; k < j->K - 1; ++k) {\n                double t", 1),
    "bf16_shift": ("(uint32_t)bits << 16", "(uint32_t)bits << 15", 1),
    "output_index": ("j->y[m * j->nrows + r] = acc;", "j->y[r * j->M + m] = acc;", 1),
    "check_signed_diff": ("double d = fabs(v - r);", "double d = v - r;", 1),
    "check_zero_base": ("if (v != 0.0)\n                ++bad;", "if (0)\n                ++bad;", 1),
    "check_nan": ("if (!isnan(v))\n                ++bad;", "if (0)\n                ++bad;", 1),
    "silu_sign": ("h[i] = gate[i] / (1.0 + exp(-gate[i])) * up[i];",
                  "h[i] = gate[i] / (1.0 + exp(gate[i])) * up[i];", 1),
    "silu_swapped": ("h[i] = gate[i] / (1.0 + exp(-gate[i])) * up[i];",
                     "h[i] = up[i] / (1.0 + exp(-up[i])) * gate[i];", 1),
    "silu_sigmoid_only": ("h[i] = gate[i] / (1.0 + exp(-gate[i])) * up[i];",
                          "h[i] = 1.0 / (1.0 + exp(-gate[i])) * up[i];", 1),
    "silu_bound_slope": ("bound[i] = 1.1 * da", "bound[i] = 0.5 * da", 1),
    "silu_bound_up_term": ("+ fabs(sg) * db;", ";", 1),
    "check_bf16_rounding": ("ldexp(fabs(r) + bound[i], -8)", "ldexp(fabs(r) + bound[i], -4)", 1),
    "quant_global_448": ("amax / 2688.0f", "amax / 448.0f", 1),
    "quant_zero_global": ("return amax == 0.0f ? 1.0f :", "return amax == 0.0f ? 0.0f :", 1),
    "quant_block_div4": ("6.0 * g * ((orc_e4m3(c)", "4.0 * g * ((orc_e4m3(c)", 1),
    "quant_e4m3_ties_odd": ("orc_e4m3(c + 1)) / 2.0);\n        if (a > lim || (a == lim && ((c + 1) & 1u) == 0))",
                            "orc_e4m3(c + 1)) / 2.0);\n        if (a > lim || (a == lim && ((c + 1) & 1u) == 1))", 1),
    "quant_e4m3_ties_up": ("orc_e4m3(c + 1)) / 2.0);\n        if (a > lim || (a == lim && ((c + 1) & 1u) == 0))",
                           "orc_e4m3(c + 1)) / 2.0);\n        if (a >= lim)", 1),
    "quant_e2m1_ties_odd": ("orc_e2m1(c + 1)) / 2.0);\n        if (a > lim || (a == lim && ((c + 1) & 1u) == 0))",
                            "orc_e2m1(c + 1)) / 2.0);\n        if (a > lim || (a == lim && ((c + 1) & 1u) == 1))", 1),
    "quant_e2m1_ties_up": ("orc_e2m1(c + 1)) / 2.0);\n        if (a > lim || (a == lim && ((c + 1) & 1u) == 0))",
                           "orc_e2m1(c + 1)) / 2.0);\n        if (a >= lim)", 1),
    "quant_e2m1_truncates": ("(orc_e2m1(c) + orc_e2m1(c + 1)) / 2.0);\n        if (a > lim || (a == lim && ((c + 1) & 1u) == 0))",
                             "orc_e2m1(c + 1));\n        if (a >= lim)", 1),
    "quant_e4m3_not_saturating": ("unsigned c = 0;\n    while (c < 0x7Eu) {",
                                  "unsigned c = 0;\n    if (a > 6.0 * g * 448.0)\n        return 0x7Fu;\n"
                                  "    while (c < 0x7Eu) {", 1),
    "quant_e2m1_not_saturating": ("while (c < 7u) {", "while (c < 6u) {", 1),
    "quant_sign_dropped": ("quant_code(a, unit) | ((bits >> 15) << 3)", "quant_code(a, unit)", 1),
    "quant_unit_without_g": ("const double unit = orc_e4m3(s) * (double)g;\n            scales",
                             "const double unit = orc_e4m3(s);\n            scales", 1),
    "quant_nibbles_swapped": ("(uint8_t)(q[0] | (q[1] << 4))", "(uint8_t)(q[1] | (q[0] << 4))", 1),
    # the limits, or the quotient itself, rounded to fp32 (an fp32 evaluation
    # of the definition, which misplaces quotients within ~2^-23 of a tie)
    "quant_scale_limit_fp32": ("const double lim = 6.0 * g * ((orc_e4m3(c) + orc_e4m3(c + 1)) / 2.0);",
                               "const double lim = (float)(6.0 * g) * (float)((orc_e4m3(c) + orc_e4m3(c + 1)) / 2.0);", 1),
    "quant_code_limit_fp32": ("const double lim = unit * ((orc_e2m1(c) + orc_e2m1(c + 1)) / 2.0);",
                              "const double lim = (float)unit * (float)((orc_e2m1(c) + orc_e2m1(c + 1)) / 2.0);", 1),
    "quant_code_quotient_fp32": ("const double lim = unit * ((orc_e2m1(c) + orc_e2m1(c + 1)) / 2.0);",
                                 "const double lim = (orc_e2m1(c) + orc_e2m1(c + 1)) / 2.0;\n"
                                 "        a = (float)a * (1.0f / (float)unit);\n        unit = 1.0;", 1),
    "quant_scale_quotient_fp32": ("const double lim = 6.0 * g * ((orc_e4m3(c) + orc_e4m3(c + 1)) / 2.0);",
                                  "const double lim = (orc_e4m3(c) + orc_e4m3(c + 1)) / 2.0;\n"
                                  "        a = ((float)a / 6.0f) / (float)g;\n        g = 1.0 / 6.0;", 1),
    "argmax_no_tolerance": ("if (!(yr[i] + tol >= floor_max)", "if (!(yr[i] >= floor_max + tol)", 1),
    "argmax_any_nan": ("if (i != first_nan || !isnan(v))", "if (!isnan(yr[i]) || !isnan(v))", 1),
    "argmax_value_unchecked": ("|| !(fabs(v - yr[i]) <= tol))", ")", 1),
    "argmax_upper_floor": ("const double lo = yr[j] - rtol * sr[j];", "const double lo = yr[j] + rtol * sr[j];", 1),
    "quant_block_amax_first": ("if (a > amax_b)\n                    amax_b = a;", "if (i == 0)\n                    amax_b = a;", 1),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new, count = MUTANTS[name]
    assert source.count(old) >= count, f"mutation site for {name} not found in oracle.c"
    mutated = source.replace(old, new, count)
    assert mutated != source
    src = tmp_path / "oracle_mut.c"
    src.write_text(mutated)
    out = str(tmp_path / f"liboracle_{name}.so")
    oracle.build(str(src), out)
    lib = oracle.load(out)
    caught = None
    for pin in pins.ALL_PINS:          # stop at the first pin that fails
        try:
            pin(lib)
        except AssertionError:
            caught = pin.__name__
            break
    assert caught, f"no pin caught the planted mistake {name}"
