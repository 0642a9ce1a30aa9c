"""Plant plausible mistakes in the oracle and check that the pins catch each.

Each mutant is the oracle's C source with one textual change (a dropped term,
a wrong sign, a wrong index, a different rounding), compiled with the same gcc
flags into a temporary library.  The pins of ``pins.py`` run against it; at
least one must fail.  The mistakes are planted in the oracle, on the CPU only.
"""


import pytest

import oracle
import pins

MUTANTS = {
    "sigmoid_sign": ("return 1.0 / (1.0 + exp(-t));", "return 1.0 / (1.0 + exp(t));"),
    "fwd_drops_alpha": ("return x * oracle_sigmoid(alpha * x);", "return x * oracle_sigmoid(x);"),
    "fwd_drops_x": ("return x * oracle_sigmoid(alpha * x);", "return oracle_sigmoid(alpha * x);"),
    "bwd_sign": ("return dy * s * (1.0 + t * one_minus_s);", "return dy * s * (1.0 - t * one_minus_s);"),
    "bwd_chain_drops_alpha": ("return dy * s * (1.0 + t * one_minus_s);",
                              "return dy * s * (1.0 + x * one_minus_s);"),
    "bwd_drops_dy": ("return dy * s * (1.0 + t * one_minus_s);", "return s * (1.0 + t * one_minus_s);"),
    "bwd_drops_one": ("return dy * s * (1.0 + t * one_minus_s);", "return dy * s * (t * one_minus_s);"),
    "bwd_one_minus_s_is_s": ("double one_minus_s = 1.0 - s;", "double one_minus_s = s;"),
    "bwd_t_without_alpha": ("    double t = alpha * x;\n    double s = oracle_sigmoid(t);",
                            "    double t = x;\n    double s = oracle_sigmoid(alpha * x);"),
    "bf16_truncates": ("double r = nearbyint(a / spacing) * spacing;",
                       "double r = floor(a / spacing) * spacing;"),
    "bf16_ties_away": ("double r = nearbyint(a / spacing) * spacing;",
                       "double r = round(a / spacing) * spacing;"),
    "bf16_wrong_spacing": ("double spacing = ldexp(1.0, k - 7);", "double spacing = ldexp(1.0, k - 8);"),
    "bf16_wrong_subnormal_floor": ("if (k < -126)\n        k = -126;", "if (k < -140)\n        k = -140;"),
    "bf16_via_f32": ("double r = nearbyint(a / spacing) * spacing;",
                     "double r = nearbyint((double)(float)a / spacing) * spacing;"),
    "f32_flushes_subnormals": ("return (float)v;", "return fabs(v) < 0x1p-126 ? (float)(0.0 * v) : (float)v;"),
    "bf16_widen_shift": ("uint32_t w = (uint32_t)bits << 16;", "uint32_t w = (uint32_t)bits << 15;"),
    "scale_drops_abs": ("*scale = fabs(dy) * s * (1.0 + fabs(t) * one_minus_s);",
                        "*scale = fabs(dy) * s * (1.0 + t * one_minus_s);"),
    "split_drops_last": ("jobs[k].end = n * (size_t)(k + 1) / (size_t)threads;",
                         "jobs[k].end = n * (size_t)(k + 1) / (size_t)threads - (k + 1 == threads);"),
    "alpha_rounded_to_int": ("oracle_job j = {ORACLE_ACT_SWISH, dtype, x, NULL, y, NULL, (double)alpha, 0, 0};",
                             "oracle_job j = {ORACLE_ACT_SWISH, dtype, x, NULL, y, NULL, (double)(int)alpha, 0, 0};"),
    # The activation family.
    "gelu_cdf_sign": ("return 0.5 * erfc(-x * kInvSqrt2);", "return 0.5 * erfc(x * kInvSqrt2);"),
    "gelu_pdf_exponent": ("return kInvSqrt2Pi * exp(-0.5 * x * x);", "return kInvSqrt2Pi * exp(-x * x);"),
    "gelu_pdf_constant": ("static const double kInvSqrt2Pi = 0.39894228040143267793994605993438187;",
                          "static const double kInvSqrt2Pi = 0.5;"),
    "gelu_grad_drops_cdf": ("g = dy * (cdf + x * pdf);", "g = dy * (x * pdf);"),
    "gelu_tanh_cubic": ("static const double kGeluTanhCubic = 0.044715;",
                        "static const double kGeluTanhCubic = 0.0447;"),
    "gelu_tanh_du": ("double du = kSqrt2OverPi * (1.0 + 3.0 * kGeluTanhCubic * x * x);",
                     "double du = kSqrt2OverPi * (1.0 + kGeluTanhCubic * x * x);"),
    "gelu_tanh_half_u": ("return x * oracle_sigmoid(2.0 * u);", "return x * oracle_sigmoid(u);"),
    "tanh_grad_not_squared": ("g = dy / (c * c);", "g = dy / c;"),
    "sigmoid_grad_s_squared": ("g = dy * oracle_sigmoid(x) * oracle_sigmoid(-x);",
                               "g = dy * oracle_sigmoid(x) * oracle_sigmoid(x);"),
    "relu_grad_drops_dy": ("g = dy * (x > 0.0 ? 1.0 : 0.0);", "g = (x > 0.0 ? 1.0 : 0.0);"),
    "leaky_fwd_drops_x": ("return x > 0.0 ? x : p * x;", "return x > 0.0 ? x : p;"),
    "leaky_grad_at_zero": ("g = dy * (x > 0.0 ? 1.0 : p);", "g = dy * (x >= 0.0 ? 1.0 : p);"),
    "gelu_scale_drops_abs": ("m = fabs(dy) * (cdf + fabs(x) * pdf);", "m = fabs(dy) * (cdf + x * pdf);"),
    # Error scales inflated: the tolerance they set would loosen.
    "swish_scale_doubled": ("*scale = fabs(dy) * s * (1.0 + fabs(t) * one_minus_s);",
                            "*scale = 2.0 * fabs(dy) * s * (1.0 + fabs(t) * one_minus_s);"),
    "gelu_scale_doubled": ("m = fabs(dy) * (cdf + fabs(x) * pdf);",
                           "m = 2.0 * fabs(dy) * (cdf + fabs(x) * pdf);"),
    "gelu_tanh_scale_doubled": ("m = fabs(dy) * (s + fabs(x) * s * c * 2.0 * du);",
                                "m = 2.0 * fabs(dy) * (s + fabs(x) * s * c * 2.0 * du);"),
    "tanh_scale_inflated": ("g = dy / (c * c);\n        m = fabs(g);",
                            "g = dy / (c * c);\n        m = 1.5 * fabs(g);"),
    "family_nan_passthrough": ("    if (isnan(x))\n        return x;\n    switch (act) {",
                               "    switch (act) {"),
    # Limits at +-inf: the value as x -> +-inf with the parameter fixed.
    "swish_limit_wrong_zero_sign": ("return t > 0.0 ? x : copysign(0.0, x);", "return t > 0.0 ? x : 0.0;"),
    "swish_grad_limit_dropped": ("    if (isinf(x)) {\n        double g = swish_grad_limit(x, dy, alpha);",
                                 "    if (0) {\n        double g = swish_grad_limit(x, dy, alpha);"),
    "gelu_limit_dropped": ("        if (isinf(x))  /* limits: x, and x Phi(x) -> -0 */\n            return x > 0.0 ? x : -0.0;\n",
                           ""),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not unique/present"
    src = tmp_path / "mutant.c"
    src.write_text(source.replace(old, new))
    lib = oracle.build(str(src), str(tmp_path / "libmutant.so"))
    o = oracle.Oracle(oracle.load(lib))
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            caught.append(pin.__name__)
            break
    assert caught, f"no pin caught mutant {name}"
