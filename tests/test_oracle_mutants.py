"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one: a dropped term, a wrong sign, a wrong or transposed
operand, a wrong index or layout, a skipped step. Each mutant keeps every
memory access in bounds."""
import os
import subprocess

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTANTS = {
    "sign_of_first_output": [("x1 * c[i] - x2 * s[i]", "x1 * c[i] + x2 * s[i]")],
    "dropped_term_second_output": [("x2 * c[i] + x1 * s[i]", "x2 * c[i]")],
    "f32_second_product_rounded_first": [("x1 * c[i] - x2 * s[i]",
                                          "x1 * c[i] - (dtype == ORACLE_F32 ? (double)(float)(x2 * s[i]) : x2 * s[i])")],
    "cos_sin_transposed": [("x1 * c[i] - x2 * s[i]", "x1 * s[i] - x2 * c[i]")],
    "operands_swapped_second_output": [("x2 * c[i] + x1 * s[i]", "x1 * c[i] + x2 * s[i]")],
    "half_split_partner": [("int64_t j2 = interleaved ? 2 * i + 1 : i + half;",
                            "int64_t j2 = interleaved ? 2 * i + 1 : R - 1 - i;")],
    "interleaved_ignored": [("int64_t j1 = interleaved ? 2 * i : i;", "int64_t j1 = i;"),
                            ("int64_t j2 = interleaved ? 2 * i + 1 : i + half;",
                             "int64_t j2 = i + half;")],
    "rank3_as_rank4": [("return ((b * S + s) * H + h) * D;", "return ((b * H + h) * S + s) * D;")],
    "tail_not_copied": [("for (int64_t j = R; j < D; ++j)", "for (int64_t j = D; j < D; ++j)")],
    "per_token_row_ignores_batch": [("row = b * S + s;", "row = s;")],
    "id_zero_out_of_range": [("in_range = row >= 0 && row < M;", "in_range = row > 0 && row < M;")],
    "out_of_range_rotated": [("in_range = row >= 0 && row < M;", "in_range = 1; if (row < 0 || row >= M) row = 0;")],
    "mrope_scale_ignored": [("(c * (double)scale)", "(c)")],
    "mrope_oob_check": [("cr.copy[i] = (unsigned char)!(p >= 0 && p < M);",
                         "cr.copy[i] = (unsigned char)!(p > 0 && p < M);")],
    "mrope_always_temporal": [("ids[(int64_t)stream[i] * B * S + b * S + s]", "ids[b * S + s]")],
    "mrope_layout1_as_layout0": [("        used[k] += 1;\n        k = (k + 1) % 3;", "        used[k] += 1;")],
    "mrope_layout_ignored": [("if (layout == 0) {", "if (1) {")],
    "cache_cos_is_sin": [("float cf = (float)cos((double)theta);", "float cf = (float)sin((double)theta);")],
    "cache_theta_not_rounded": [("float theta = (float)((double)pf * (double)inv_freq_i);",
                                 "double theta = (double)pf * (double)inv_freq_i;")],
    "cache_scaling_ignored": [("float cs = (float)((double)cf * (double)scaling);", "float cs = cf;")],
    "f16_round_down": [("nearbyint(a / quantum)", "floor(a / quantum)")],
    "f16_subnormal_scale": [("v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);")],
    "bf16_decode_exponent": [("v = ldexp((double)(128 + m), e - 134);", "v = ldexp((double)(128 + m), e - 133);")],
    "bf16_subnormal_bound": [("if (r < ldexp(1.0, -126))", "if (r < ldexp(1.0, -127))")],
    "bf16_fraction_bits": [("ldexp(r, 7 - E) - 128.0", "ldexp(r, 7 - E) - 127.0")],
    "bf16_stored_as_f16": [("((uint16_t*)p)[idx] = oracle_f64_to_bf16(v);",
                            "((uint16_t*)p)[idx] = oracle_f64_to_f16(v);")],
    "kv_past_without_minus_s": [("(int64_t)key_total_sequence_lengths[b] - S;", "(int64_t)key_total_sequence_lengths[b];")],
    "kv_prompt_ignored": [("int prompt = total_sequence_length == S;", "int prompt = 0;")],
    "kv_cache_head_major_swapped": [("int64_t dst = ((b * Hk + h) * Smax + p) * D;",
                                     "int64_t dst = ((h * B + b) * Smax + p) * D;")],
    "kv_packed_key_value_swapped": [("int64_t k0 = packed ? H * D : 0;", "int64_t k0 = packed ? (H + Hk) * D : 0;"),
                                    ("int64_t v0 = packed ? (H + Hk) * D : 0;", "int64_t v0 = packed ? H * D : 0;")],
    "kv_row_bound_off_by_one": [("if (p < 0 || p >= Smax)", "if (p < 0 || p > Smax - 2)")],
    "kv_value_not_written": [("                    copy_elem_to(dtype, vsrc, tok * kw + v0 + h * D + j,\n                                 past_value, dst + j);",
                              "                    ;")],
    "norm_sum_not_mean": [("1.0 / sqrt(ss / (double)D + eps)", "1.0 / sqrt(ss + eps)")],
    "norm_epsilon_ignored": [("1.0 / sqrt(ss / (double)D + eps)", "1.0 / sqrt(ss / (double)D)")],
    "norm_no_square_root": [("1.0 / sqrt(ss / (double)D + eps)", "1.0 / (ss / (double)D + eps)")],
    "norm_weight_ignored": [("z[j] = load_elem(dtype, x, off + j) * inv_rms * load_elem(dtype, w, j);",
                             "z[j] = load_elem(dtype, x, off + j) * inv_rms;")],
    "norm_k_uses_q_weight": [("norm_row(dtype, k, off, k_weight, D, (double)epsilon, z);",
                              "norm_row(dtype, k, off, q_weight, D, (double)epsilon, z);")],
    "norm_tail_not_normalised": [("        store_elem(dtype, y, off + j, z[j]);\n}",
                                  "        store_elem(dtype, y, off + j, z[j] / z[j] * 0.0 + 1.0);\n}")],
    "kv_norm_value_normalised": [("                    copy_elem_to(dtype, vsrc, tok * kw + v0 + h * D + j,\n                                 past_value, dst + j);",
                                  "                    store_elem(dtype, past_value, dst + j, z[j]);")],
    "kv_norm_k_uses_q_weight": [("norm_row(dtype, ksrc, tok * kw + k0 + h * D, k_weight, D,",
                                 "norm_row(dtype, ksrc, tok * kw + k0 + h * D, q_weight, D,")],
    "inv_freq_exponent": [("-2.0 * (double)i / (double)rotary_dim", "-1.0 * (double)i / (double)rotary_dim")],
    "onthefly_uses_position_zero": [("coefficient(dtype, p, inv_freq[i], scaling, &cr.c[i], &cr.s[i]);",
                                     "coefficient(dtype, 0, inv_freq[i], scaling, &cr.c[i], &cr.s[i]);")],
}


def _build_mutant(name, edits, tmpdir):
    with open(oracle.SOURCE_PATH) as f:
        src = f.read()
    for old, new in edits:
        assert src.count(old) >= 1, "mutation %s: pattern not found: %r" % (name, old)
        src = src.replace(old, new)
    c_path = os.path.join(tmpdir, "mutant_%s.c" % name)
    so_path = os.path.join(tmpdir, "libmutant_%s.so" % name)
    with open(c_path, "w") as f:
        f.write(src)
    hdr_dir = os.path.dirname(oracle.SOURCE_PATH)
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-w",
                           "-fno-fast-math", "-ffp-contract=off", "-I", hdr_dir,
                           c_path, "-o", so_path, "-lm"])
    return so_path


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    so = _build_mutant(name, MUTANTS[name], str(tmp_path))
    orc = oracle.Oracle(so)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError) as e:
            caught.append(pin.__name__)
    assert caught, "no pin catches the planted mistake %s" % name
