"""The pins have teeth: plausible mistakes planted in copies of the oracle's
C source (on the CPU, in a temporary directory) must each fail a pin.

Each mutant is one textual edit of ``oracle/oracle.c`` (a dropped term, a
wrong sign, divisor, index or operand), compiled with gcc to a private
shared library.  None of the edits reads out of bounds.
"""
import os
import shutil

import pytest

import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "rms_divisor_n_minus_1": ("double mean_sq = sum_sq / (double)width;",
                              "double mean_sq = sum_sq / (double)(width > 1 ? width - 1 : 1);"),
    "rms_dropped_eps": ("double root = sqrt(mean_sq + e);", "double root = sqrt(mean_sq);"),
    "rms_eps_outside_root": ("double root = sqrt(mean_sq + e);",
                             "double root = sqrt(mean_sq) + e;"),
    "rms_sum_not_squared": ("sum_sq += v * v;", "sum_sq += v * (v < 0 ? -v : v);"),
    "rms_multiply_by_root": ("y[r * width + j] = v / root * widen(w, dtype, j);",
                             "y[r * width + j] = v * root * widen(w, dtype, j);"),
    "rms_weight_reversed": ("y[r * width + j] = v / root * widen(w, dtype, j);",
                            "y[r * width + j] = v / root * widen(w, dtype, width - 1 - j);"),
    "rms_no_weight": ("y[r * width + j] = v / root * widen(w, dtype, j);",
                      "y[r * width + j] = v / root;"),
    "layer_mean_divisor": ("double mean = sum / (double)width;",
                           "double mean = sum / (double)(width + 1);"),
    "layer_var_unbiased": ("double var = sum_dev_sq / (double)width;",
                           "double var = sum_dev_sq / (double)(width > 1 ? width - 1 : 1);"),
    "layer_dropped_eps": ("double root = sqrt(var + e);", "double root = sqrt(var);"),
    "layer_bias_sign": ("y[r * width + j] = d / root * widen(w, dtype, j) + bias;",
                        "y[r * width + j] = d / root * widen(w, dtype, j) - bias;"),
    "layer_no_centering": ("double d = widen(x, dtype, r * width + j) - mean;\n"
                           "            double bias",
                           "double d = widen(x, dtype, r * width + j);\n"
                           "            double bias"),
    "layer_var_of_raw_x": ("sum_dev_sq += d * d;",
                           "sum_dev_sq += (d + mean) * (d + mean);"),
    "layer_bias_reversed": ("double bias = b ? widen(b, dtype, j) : 0.0;",
                            "double bias = b ? widen(b, dtype, width - 1 - j) : 0.0;"),
    "bf16_decode_shift": ("uint32_t bits = ((uint32_t)h[i]) << 16;",
                          "uint32_t bits = ((uint32_t)h[i]) << 15;"),
    "bf16_decode_low_half": ("uint32_t bits = ((uint32_t)h[i]) << 16;",
                             "uint32_t bits = ((uint32_t)h[i]) << 16 | 0x8000u;"),
    "dual_swapped_weights": ("oracle_rms(k, kw, dtype, k_rows, head_dim, eps, ky);",
                             "oracle_rms(k, qw, dtype, k_rows, head_dim, eps, ky);"),
    "dual_eps_dropped_for_keys": ("oracle_rms(k, kw, dtype, k_rows, head_dim, eps, ky);",
                                  "oracle_rms(k, kw, dtype, k_rows, head_dim, 0.0f, ky);"),
    "f16_exponent_bias": ("v = ldexp((double)(fraction | 0x400), exponent - 25);",
                          "v = ldexp((double)(fraction | 0x400), exponent - 24);"),
    "f16_no_implicit_bit": ("v = ldexp((double)(fraction | 0x400), exponent - 25);",
                            "v = ldexp((double)(fraction), exponent - 25);"),
    "f16_subnormal_scale": ("v = ldexp((double)fraction, -24);",
                            "v = ldexp((double)fraction, -25);"),
    "f16_sign_dropped": ("return sign ? -v : v;", "return v;"),
    "rope_sign": ("x[a] = xa * c - xb * s;", "x[a] = xa * c + xb * s;"),
    "rope_cos_sin_swapped": ("double c = cos(theta), s = sin(theta);",
                             "double c = sin(theta), s = cos(theta);"),
    "rope_no_offset": ("const double pos = (double)(offset + r / heads);",
                       "const double pos = (double)(r / heads);"),
    "rope_position_per_row": ("const double pos = (double)(offset + r / heads);",
                              "const double pos = (double)(offset + r);"),
    "rope_exponent_head_dim": ("pow((double)base, -2.0 * (double)i / (double)dims)",
                               "pow((double)base, -2.0 * (double)i / (double)head_dim)"),
    "rope_exponent_no_two": ("pow((double)base, -2.0 * (double)i / (double)dims)",
                             "pow((double)base, -1.0 * (double)i / (double)dims)"),
    "rope_no_scale": ("double theta = pos * (double)scale * inv_freq;",
                      "double theta = pos * inv_freq;"),
    "rope_split_pairs_adjacent": ("int64_t b = traditional ? 2 * i + 1 : i + half;",
                                  "int64_t b = traditional ? 2 * i + 1 : half - 1 - i + half;"),
    "rope_interleave_as_split": ("int64_t a = traditional ? 2 * i : i;",
                                 "int64_t a = i;"),
    "rope_freqs_ignored": ("double inv_freq = freqs ? (double)freqs[i]",
                           "double inv_freq = 0 ? (double)freqs[i]"),
    "dual_rope_keys_use_query_heads": (
        "oracle_rope_rows(ky, tokens * k_heads, k_heads,",
        "oracle_rope_rows(ky, tokens * k_heads, q_heads,"),
    "swiglu_gate_sign": ("double silu = gate / (1.0 + exp(-gate));",
                         "double silu = gate / (1.0 + exp(gate));"),
    "swiglu_sigmoid_only": ("double silu = gate / (1.0 + exp(-gate));",
                            "double silu = 1.0 / (1.0 + exp(-gate));"),
    "swiglu_gate_reads_x": ("double gate = widen(g, dtype, i);",
                            "double gate = widen(x, dtype, i);"),
    "swiglu_gate_dropped": ("y[i] = y[i] * silu;", "y[i] = y[i] * 1.0;"),
    "swiglu_gate_added": ("y[i] = y[i] * silu;", "y[i] = y[i] + silu;"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, source, name):
    old, new = MUTANTS[name]
    assert source.count(old) >= 1, f"mutation site for {name} not found"
    src = tmp_path / "oracle_mutant.c"
    src.write_text(source.replace(old, new, 1))
    lib = oracle.build(str(src), str(tmp_path / f"lib_{name}.so"))
    mutant = oracle.Oracle(lib)
    failures = []
    for pin in oracle_pins.PINS:
        try:
            pin(mutant)
        except AssertionError as e:
            failures.append(f"{pin.__name__}: {e}")
    assert failures, f"mutant {name} passed every pin"
