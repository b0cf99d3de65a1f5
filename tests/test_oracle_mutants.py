"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pins in test_oracle.py catch each one.  The real oracle is never
modified: each mutant is a separately compiled copy loaded in its place for
the duration of one check.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
import tests.test_oracle as pins

SRC = open(oracle.SRC).read()

MUTANTS = {
    "drops_last_term": ("for (int64_t k = 0; k < K; ++k)\n            s += oracle_bf16_to_f64(xr[k]) * oracle_bf16_to_f64",
                        "for (int64_t k = 0; k + 1 < K; ++k)\n            s += oracle_bf16_to_f64(xr[k]) * oracle_bf16_to_f64"),
    "w32_drops_last_term": ("for (int64_t k = 0; k < K; ++k)\n            s += oracle_bf16_to_f64(xr[k]) * (double)",
                            "for (int64_t k = 0; k + 1 < K; ++k)\n            s += oracle_bf16_to_f64(xr[k]) * (double)"),
    "transposed_operand": ("const uint16_t *wr = W + n * K;", "const uint16_t *wr = W + m * K;"),
    "bias_sign": ("s += oracle_bf16_to_f64(bias[n]);", "s -= oracle_bf16_to_f64(bias[n]);"),
    "bias_wrong_index": ("s += oracle_bf16_to_f64(bias[n]);", "s += oracle_bf16_to_f64(bias[0]);"),
    "gelu_constant": ("(s + 0.044715 * s", "(s + 0.04715 * s"),
    "gelu_half": ("return 0.5 * s * (1.0 + tanh", "return s * (1.0 + tanh"),
    "rounding_truncates": ("double r = nearbyint(units);", "double r = floor(units);"),
    "rounding_ties_away": ("double r = nearbyint(units);", "double r = round(units);"),
    "subnormal_spacing": ("if (q < -133) q = -133;", "if (q < -126) q = -126;"),
    "overflow_saturates": ("if (v >= 0x1p128) return (uint16_t)(sign | 0x7F80u);",
                           "if (v >= 0x1p128) return (uint16_t)(sign | 0x7F7Fu);"),
    "decode_shift": ("(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    "fraction_bits": ("int q = (e - 1) - 7;", "int q = (e - 1) - 8;"),
    "hilo_residual_sign": ("double r = x - oracle_bf16_to_f64(h);", "double r = oracle_bf16_to_f64(h) - x;"),
    "hilo_hi_truncates": ("uint16_t h = oracle_f64_to_bf16(x);",
                          "float xf_ = (float)x; uint32_t u_; memcpy(&u_, &xf_, 4); uint16_t h = (uint16_t)(u_ >> 16);"),
    "hilo_lo_truncates": ("lo[i] = oracle_f64_to_bf16(r);",
                          "float rf_ = (float)r; uint32_t v_; memcpy(&v_, &rf_, 4); lo[i] = (uint16_t)(v_ >> 16);"),
    "w32_weights_rounded_to_bf16": ("s += oracle_bf16_to_f64(xr[k]) * (double)wr[k];",
                                    "s += oracle_bf16_to_f64(xr[k]) * oracle_bf16_to_f64(oracle_f64_to_bf16(wr[k]));"),
    "w32_transposed_operand": ("const float *wr = W32 + n * K;", "const float *wr = W32 + m * K;"),
}

PIN_TESTS = [
    lambda: [pins.test_worked_examples_exact(c) for c in pins.golden()["projections"]],
    pins.test_reduction_split_partials,
    pins.test_storage_and_transpose_identity,
    pins.test_matches_numpy_float64_matmul,
    pins.test_exact_rational_brute_force_tiny,
    pins.test_integer_inputs_exact_with_bias,
    pins.test_decode_all_bf16_patterns,
    pins.test_bf16_page_values,
    pins.test_bf16_direct_rounding_avoids_double_rounding,
    pins.test_bf16_encode_vs_bit_trick_on_fp32_inputs,
    pins.test_bf16_encode_vs_exact_rationals_on_doubles,
    pins.test_gelu_tanh_vs_torch_float64,
    pins.test_gelu_identities_and_limits,
    pins.test_epilogue_order_bias_then_gelu,
    pins.test_hilo_page_example,
    pins.test_hilo_vs_bit_trick,
    pins.test_hilo_error_bounds,
    pins.test_hilo_recovers_constructed_pairs,
    pins.test_w32_matches_numpy_float64_matmul,
    pins.test_w32_exact_rationals_and_bias,
    pins.test_w32_agrees_with_bf16_oracle_on_bf16_weights,
]


def _build_mutant(tmp_path, name, old, new):
    assert SRC.count(old) >= 1, "mutation site vanished: " + name
    src = tmp_path / (name + ".c")
    src.write_text(SRC.replace(old, new, 1))
    so = tmp_path / (name + ".so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", str(src),
                    "-o", str(so), "-lm"], check=True)
    return str(so)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name, monkeypatch):
    old, new = MUTANTS[name]
    so = _build_mutant(tmp_path, name, old, new)
    real = oracle.lib()
    # load the mutant with the real library's signatures
    mut = ctypes.CDLL(so)
    for fn in ("oracle_proj_f64", "oracle_proj_f64_at", "oracle_round_out", "oracle_f64_to_bf16_array",
               "oracle_bf16_to_f64_array", "oracle_gelu_tanh_array", "oracle_proj_f64_w32",
               "oracle_hilo_split"):
        f, g = getattr(mut, fn), getattr(real, fn)
        f.argtypes, f.restype = g.argtypes, g.restype
    monkeypatch.setattr(oracle, "_lib", mut)
    caught = 0
    for t in PIN_TESTS:
        try:
            t()
        except (AssertionError, ValueError):
            caught += 1
    assert caught > 0, "no pin caught mutant " + name
