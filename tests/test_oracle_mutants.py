"""The oracle's pins must catch plausible mistakes.

Each mutant is a copy of ``oracle/oracle.c`` with one mistake planted by text
substitution (the committed oracle is never changed), compiled with gcc into a
temporary directory.  The test requires that at least one check of
``oracle_checks.ALL_CHECKS`` fails on every mutant.  No mutant reads or writes
out of bounds, so they run in-process.
"""

import os

import pytest

import oracle
import oracle_checks

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "xnor_sign_zero_negative": [("return (v < 0.0f) ? -1 : 1;", "return (v <= 0.0f) ? -1 : 1;")],
    "and_sign_zero_negative": [("return (v < 0.0f) ? 0 : 1;", "return (v <= 0.0f) ? 0 : 1;")],
    "msb_first_bit_order": [(">> (c % 32)", ">> (31 - c % 32)")],
    "and_weights_pm1": [("if (type == ORACLE_AND) return bit;",
                         "if (type == ORACLE_AND) return bit ? 1 : -1;")],
    "xnor_weight_polarity": [("return bit ? 1 : -1;", "return bit ? -1 : 1;")],
    "padding_clamps": [("if (ix < 0 || ix >= in_w) continue; /* padded tap: nothing */",
                        "if (ix < 0 || ix >= in_w) ix = ix < 0 ? 0 : in_w - 1;")],
    "padding_row_clamps": [("if (iy < 0 || iy >= in_h) continue; /* padded tap: nothing */",
                            "if (iy < 0 || iy >= in_h) iy = iy < 0 ? 0 : in_h - 1;")],
    "beta_divides_by_valid_taps": [("b = sum / (double)(use_beta == 2 ? valid : kernel_h * kernel_w);",
                                    "b = sum / (double)valid;")],
    "valid_tap_beta_divides_by_window": [("b = sum / (double)(use_beta == 2 ? valid : kernel_h * kernel_w);",
                                          "b = sum / (double)(kernel_h * kernel_w);")],
    "valid_tap_count_includes_padding": [("                            ++valid;\n", ""),
                                         ("                    int valid = 0;\n",
                                          "                    int valid = kernel_h * kernel_w;\n")],
    "affine_offset_then_scale": [("v = fmaf(v, s, b);", "v = (v + b) * s;")],
    "affine_two_roundings": [("v = fmaf(v, s, b);", "v = (float)(v * s) + b;")],
    "a_map_over_word_width": [("am[p] = sum / (double)in_c;", "am[p] = sum / (double)(words * 32);")],
    "a_map_before_affine": [("sum += fabs(xd[p * in_c + c]);", "sum += fabs((double)x[p * in_c + c]);")],
    "ceil_mode_output_size": [("return (in + pad + pad_end - k) / stride + 1;",
                               "return (in + pad + pad_end - k + stride - 1) / stride + 1;")],
    "trailing_pad_is_leading": [("return (in + pad + pad_end - k) / stride + 1;",
                                 "return (in + 2 * pad - k) / stride + 1;")],
    "epilogue_drops_beta": [("double r = v * scale * bw[((long)i * out_h + oy) * out_w + ox] + bias;",
                             "double r = v * scale + bias;")],
    "relu_clamps_positive": [("case ORACLE_NEURON_RELU: return r < 0.0 ? 0.0 : r;",
                              "case ORACLE_NEURON_RELU: return r > 0.0 ? 0.0 : r;")],
    "sigmoid_sign": [("return 1.0 / (1.0 + exp(-r));", "return 1.0 / (1.0 + exp(r));")],
    "tanh_drops_scale": [("return a * tanh(b * r);", "return tanh(b * r);")],
    "softplus_drops_max": [("return a * (fmax(z, 0.0) + log1p(exp(-fabs(z))));",
                            "return a * log1p(exp(-fabs(z)));")],
    "elu_scales_positive": [("return r < 0.0 ? a * expm1(r) : r;", "return r < 0.0 ? a * expm1(r) : a * r;")],
    "clamp_bounds_swapped": [("return fmin(fmax(r, a), b);", "return fmin(fmax(r, b), a);")],
    "leaky_slope_on_positive": [("return r < 0.0 ? a * r : r;", "return r < 0.0 ? r : a * r;")],
    "hard_sigmoid_no_upper_clamp": [("return fmin(fmax(a * r + b, 0.0), 1.0);", "return fmax(a * r + b, 0.0);")],
    "softsign_drops_abs": [("return r / (1.0 + fabs(r));", "return r / (1.0 + r);")],
    "missing_bias_is_one": [("(double)output_bias[co] : 0.0;", "(double)output_bias[co] : 1.0;")],
    "scale_value_ignored": [("(double)output_scale[co] : (double)scale_value;",
                             "(double)output_scale[co] : 1.0;")],
    "flipped_kernel": [("weight_value(weight_bits, words, co, ky, kx, kernel_h, kernel_w, c, type)",
                        "weight_value(weight_bits, words, co, kernel_h - 1 - ky, kernel_w - 1 - kx,"
                        " kernel_h, kernel_w, c, type)")],
    "stride_ignored_in_window": [
        ("int iy = oy * stride_h - pad_h + ky;\n                        if (iy < 0 || iy >= in_h) continue; /* padded",
         "int iy = oy - pad_h + ky;\n                        if (iy < 0 || iy >= in_h) continue; /* padded")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new, 1)
    path = tmp_path / "mutant.c"
    path.write_text(src)
    so = str(tmp_path / f"libmutant_{name}.so")
    oracle.build(str(path), so)
    lib = oracle.load(so)
    failed = []
    for check in oracle_checks.ALL_CHECKS:
        try:
            check(lib)
        except (AssertionError, ValueError):
            failed.append(check.__name__)
            break
    assert failed, f"no pin catches mutant {name}"
