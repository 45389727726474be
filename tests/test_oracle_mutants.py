"""Plant plausible mistakes in copies of the oracle (on the CPU) and require
the pin suite to catch each one, so that a pass of the pins means something.

Each mutant is one textual substitution in ``oracle/mxq_oracle.c``; the test
asserts the original text occurs exactly once, so a mutant cannot silently
stop applying when the oracle is edited.
"""
import os
import subprocess

import pytest

import oracle
from pins import ALL_PINS

MUTANTS = {
    "transposed_block": ("acc += xs[k] * R[k][n];", "acc += xs[k] * R[n][k];"),
    "scale_off_by_one": ("int e = (q - 1) - 2;", "int e = (q - 1) - 1;"),
    "log2_ceil": ("int e = (q - 1) - 2;", "int e = q - 2;"),
    "tie_up_at_quarter": ("if (a <= 0.25) return 0;", "if (a < 0.25) return 0;"),
    "tie_down_at_three_quarters": ("if (a < 0.75) return 1;", "if (a <= 0.75) return 1;"),
    "tie_up_at_2p5": ("if (a <= 2.5) return 4;", "if (a < 2.5) return 4;"),
    "tie_down_at_3p5": ("if (a < 3.5) return 5;", "if (a <= 3.5) return 5;"),
    "no_saturation_band": ("if (a <= 5.0) return 6;", "if (a <= 6.0) return 6;"),
    "negative_zero_kept": ("int neg = signbit(v) && mag != 0;", "int neg = signbit(v);"),
    "nibbles_swapped": ("codes16[j] = (uint8_t)(c[2 * j] | (c[2 * j + 1] << 4));",
                        "codes16[j] = (uint8_t)(c[2 * j + 1] | (c[2 * j] << 4));"),
    "clamp_low_wrong": ("if (e < -127) e = -127;", "if (e < -126) e = -126;"),
    "clamp_high_wrong": ("if (e > 127) e = 127;", "if (e > 126) e = 126;"),
    "amax_skips_first": ("for (int n = 0; n < GROUP; ++n) {\n        double a = fabs(y[n]);",
                         "for (int n = 1; n < GROUP; ++n) {\n        double a = fabs(y[n]);"),
    "dequant_exponent_bias": ("ldexp(mag, S - 127)", "ldexp(mag, S - 126)"),
    "dequant_sign_bit": ("out[t * channels + c] = (code & 8) ? -v : v;",
                         "out[t * channels + c] = (code & 4) ? -v : v;"),
    "dequant_nibble_order": ("int code = (c & 1) ? (byte >> 4) : (byte & 0xf);",
                             "int code = (c & 1) ? (byte & 0xf) : (byte >> 4);"),
    "fp16_exponent_bias": ("ex - 25);", "ex - 24);"),
    "fp16_subnormal_scale": ("ldexp((double)fr, -24);", "ldexp((double)fr, -25);"),
    "quant_ignores_stride": ("y[k] = load_elem(x, dtype, t * stride + g * GROUP + k);",
                             "y[k] = load_elem(x, dtype, t * channels + g * GROUP + k);"),
    "rotate_ignores_stride": ("double v = load_elem(x, dtype, t * stride + c);",
                              "double v = load_elem(x, dtype, t * channels + c);"),
    "norm_eps_outside_root": ("1.0 / sqrt(sq / (double)channels + eps)",
                              "1.0 / (sqrt(sq / (double)channels) + eps)"),
    "norm_no_root": ("1.0 / sqrt(sq / (double)channels + eps)", "1.0 / (sq / (double)channels + eps)"),
    "norm_unbiased_variance": ("sqrt(sq / (double)channels + eps)", "sqrt(sq / (double)(channels - 1) + eps)"),
    "layernorm_mean_ignored": ("mu = sum / (double)channels;", "mu = 0.0 * sum;"),
    "norm_gamma_ignored": ("double a = n * (double)gamma[c] +", "double a = n +"),
    "norm_beta_before_gamma": ("double a = n * (double)gamma[c] + (beta ? (double)beta[c] : 0.0);",
                               "double a = (n + (beta ? (double)beta[c] : 0.0)) * (double)gamma[c];"),
    "block_groups_misaligned": ("encode_group(row + g * GROUP,", "encode_group(row + g * GROUP + (g > 0),"),
    "dropped_term": ("for (int k = 0; k < B; ++k)\n            acc +=",
                     "for (int k = 1; k < B; ++k)\n            acc +="),
    "lambda_multiplies": ("return lambda ? v / (double)lambda[c] : v;",
                          "return lambda ? v * (double)lambda[c] : v;"),
    "lambda_wrong_channel": ("xs[k] = smooth(v, lambda, c);", "xs[k] = smooth(v, lambda, k);"),
    "norm_smooth_before_beta": ("xs[k] = smooth(a, lambda, c);",
                                "xs[k] = smooth(n * (double)gamma[c], lambda, c) + (beta ? (double)beta[c] : 0.0);"),
    "norm_lambda_ignored": ("xs[k] = smooth(a, lambda, c);", "xs[k] = a;"),
    "block_lambda_ignored": ("xs[k] = smooth(load_elem(x, dtype, t * stride + c), lambda, c);",
                             "xs[k] = smooth(load_elem(x, dtype, t * stride + c), NULL, c);"),
    "block_load_transposed": ("R[k][n] = load_elem(r, r_dtype, k * block + n);",
                              "R[k][n] = load_elem(r, r_dtype, n * block + k);"),
}


@pytest.fixture(scope="module")
def source():
    return open(oracle.SOURCE).read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not unique"
    src = tmp_path / f"mut_{name}.c"
    src.write_text(source.replace(old, new))
    lib = str(tmp_path / f"libmut_{name}.so")
    subprocess.run(oracle.build_command(str(src), lib), check=True)
    orc = oracle.Oracle(lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"
