"""Planted mistakes in the oracle must be caught by its pins.

Each case copies ``oracle/moe_oracle.c`` with one plausible mistake (a dropped
term, a wrong sign, index or offset, a transposed operand, a broken tie rule),
builds it into a temporary directory with the same gcc line, binds the
``oracle`` module to it and requires at least one pin of ``oracle_pins`` to
fail.  CPU only; the real oracle is restored afterwards.
"""
import os

import pytest

import oracle
import oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "moe_oracle.c")

# (name, original text, planted text)
MUTANTS = [
    ("nibble_order_swapped", "(row[k / 2] >> (4 * (k & 1)))", "(row[k / 2] >> (4 * (1 - (k & 1))))"),
    ("sym_offset_7", "(double)(code - 8)", "(double)(code - 7)"),
    ("asym_min_sign", "+ oracle_f16_value(sm[2 * gi + 1])", "- oracle_f16_value(sm[2 * gi + 1])"),
    ("asym_scale_min_swapped", "(double)code * oracle_f16_value(sm[2 * gi]) + oracle_f16_value(sm[2 * gi + 1])",
     "(double)code * oracle_f16_value(sm[2 * gi + 1]) + oracle_f16_value(sm[2 * gi])"),
    ("f16_subnormal_exponent", "ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    ("f16_bias", "ldexp((double)(f | 0x400), e - 25)", "ldexp((double)(f | 0x400), e - 24)"),
    ("bf16_ties_away", "(dropped == 0x8000u && (kept & 1u))", "(dropped == 0x8000u)"),
    ("router_transposed", "oracle_bf16_value(wr[(size_t)e * H + h])", "oracle_bf16_value(wr[(size_t)h * E + e])"),
    ("router_bias_dropped", "acc += (double)bias[e];", "acc += 0.0;"),
    ("topk_ties_to_higher", "if (best < 0 || v > bv)", "if (best < 0 || v >= bv)"),
    ("topk_nan_unmapped", "return isnan(v) ? -INFINITY : v;", "return v;"),
    ("topk_nan_first", "return isnan(v) ? -INFINITY : v;", "return isnan(v) ? INFINITY : v;"),
    ("topk_signed_zero_ordered", "return isnan(v) ? -INFINITY : v;",
     "return isnan(v) ? -INFINITY : (v == 0.0 && signbit(v) ? -1e-300 : v);"),
    ("gates_not_normalised", "- l0) / den);", "- l0));"),
    ("gates_no_shift_to_first", "exp(logit_value(l[idx[t * k + i]]) - l0) / den", "exp(logit_value(l[idx[t * k + i]])) / den"),
    ("group_unstable", "for (int64_t p = 0; p < P; p++) {\n        int e = idx[p];",
     "for (int64_t p = P - 1; p >= 0; p--) {\n        int e = idx[p];"),
    ("silu_sign", "return a / (1.0 + exp(-a));", "return a / (1.0 + exp(a));"),
    ("gate_up_swapped", "h[n] = silu(a) * b;", "h[n] = silu(b) * a;"),
    ("down_transposed", "acc += wd[(size_t)d * I + n] * h[n];", "acc += wd[(size_t)n * H + d] * h[n];"),
    ("combine_ignores_gate", "acc += (double)gate[t * k + i] * o[", "acc += 1.0 * o["),
    ("combine_one_slot", "for (int i = 0; i < k; i++)\n                acc += (double)gate",
     "for (int i = 0; i < 1; i++)\n                acc += (double)gate"),
    ("int8_unsigned", "* (double)q[(size_t)n * K + k];", "* (double)(uint8_t)q[(size_t)n * K + k];"),
    ("int8_first_group_scale", "s[(size_t)n * (K / 128) + k / 128]", "s[(size_t)n * (K / 128)]"),
    ("shared_silu_on_up", "h[n] = b * silu(a);", "h[n] = a * silu(b);"),
    ("shared_down_transposed", "acc += h[n] * wd[(size_t)d * I + n];", "acc += h[n] * wd[(size_t)n * H + d];"),
    ("shared_y_in_dropped", "double acc = y_in ? (double)y_in[(size_t)j * H + d] : 0.0;", "double acc = 0.0;"),
    ("e4m3_bias_8", "ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 11)"),
    ("e4m3_subnormal_scale", "v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    ("e4m3_sign_dropped", "return sgn ? -v : v;", "return v;"),
    ("fp8_block_row_ignored", "bs[(size_t)(n / 128) * (K / 128) + k / 128]", "bs[(size_t)(k / 128)]"),
    ("e2m1_sign_dropped", "return (sgn ? -1.0 : 1.0) * v;", "return v;"),
    ("e2m1_bias_2", "ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e - 2)"),
    ("e2m1_subnormal_quarter", "double v = e == 0 ? 0.5 * m :", "double v = e == 0 ? 0.25 * m :"),
    ("nvfp4_block_of_32", "sb[(size_t)n * (K / 16) + k / 16]", "sb[(size_t)n * (K / 16) + k / 32]"),
    ("nvfp4_global_dropped", "double ggu = fmt == ORACLE_FMT_NVFP4 ? (double)glob[2 * e] : 1.0;",
     "double ggu = 1.0;"),
    ("residual_truncates", "out[i] = oracle_bf16_round(s);", "out[i] = (uint16_t)(oracle_bf16_round(s) & 0xfffe);"),
]


@pytest.mark.parametrize("name,orig,planted", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, orc, name, orig, planted):
    text = open(SRC).read()
    assert text.count(orig) == 1, f"mutation site for {name} not unique"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(orig, planted))
    lib = oracle.compile_source(str(src), str(tmp_path / "libmutant.so"))
    prev = oracle.use_library(lib)
    caught = []
    try:
        for pin in pins.ALL_PINS:
            try:
                pin()
            except AssertionError:
                caught.append(pin.__name__)
    finally:
        oracle._lib = prev
    assert caught, f"no pin catches the planted mistake {name}"
