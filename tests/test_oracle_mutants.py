"""Each mutant is a copy of oracle.c with one plausible mistake planted (a
dropped term, a wrong sign, index or operand, a rounding slip). Each is
built on the CPU and run through the pins; every mutant must fail at least
one pin, which shows the pins can see that kind of mistake. Mutants are
chosen so that none of them can index outside its buffers."""
import os

import pytest

import oracle
from oracle_pins import PINS

MUTANTS = {
    "eps_dropped": ("1.0 / sqrt(ms + eps)", "1.0 / sqrt(ms)"),
    "eps_outside_sqrt": ("1.0 / sqrt(ms + eps)", "1.0 / sqrt(ms) + eps"),
    "sum_not_mean": ("double ms = sum_sq / (double)d;", "double ms = sum_sq;"),
    "weight_dropped": ("* r * load(w, j, dtype);", "* r;"),
    "weight_reversed": ("* r * load(w, j, dtype);", "* r * load(w, d - 1 - j, dtype);"),
    "residual_not_stored": ("            store(x, r * x_stride + j, s, dtype);\n", ""),
    "rope_sign": ("out[i] = x1 * c - x2 * s;", "out[i] = x1 * c + x2 * s;"),
    "rope_sin_cos_swapped": ("double c = cos(a), s = sin(a);", "double c = sin(a), s = cos(a);"),
    "rope_adjacent_pairs": ("double x2 = x[i + half];", "double x2 = x[i ^ 1];"),
    "rope_frequency_exponent": ("pow(base, -2.0 * (double)i / (double)d)",
                                "pow(base, -1.0 * (double)i / (double)d)"),
    "rope_k_head_stride": ("rope_head(k, t * k_ts + h * k_hs,", "rope_head(k, t * k_ts + 0 * k_hs,"),
    "qknorm_k_head_stride": ("rms_norm_head(k, t * k_ts + h * k_hs,", "rms_norm_head(k, t * k_ts + 0 * k_hs,"),
    "kv_halves_swapped": ("(((0 * num_blocks + block)", "(((1 * num_blocks + block)"),
    "skip_zero_slot": ("if (slot < 0 || slot >= n_slots) continue;",
                       "if (slot <= 0 || slot >= n_slots) continue;"),
    "silu_exp_sign": ("1.0 / (1.0 + exp(-g))", "1.0 / (1.0 + exp(g))"),
    "swiglu_up_dropped": ("out[r * out_stride + c] = g * sigmoid * u;",
                          "out[r * out_stride + c] = g * sigmoid;"),
    "bf16_double_rounding": ("double n = rint(a / q);", "double n = rint((double)(float)a / q);"),
    "bf16_truncation": ("double n = rint(a / q);", "double n = floor(a / q);"),
    "qknorm_eps_dropped": ("double r = 1.0 / sqrt(sum_sq / (double)d + eps);",
                           "double r = 1.0 / sqrt(sum_sq / (double)d);"),
    "qknorm_weight_of_q_for_k": ("rms_norm_head(k, t * k_ts + h * k_hs, k_w,",
                                 "rms_norm_head(k, t * k_ts + h * k_hs, q_w,"),
    "qknorm_weight_reversed": ("n[e] = load(x, x_off + e, dtype) * r * load(w, e, dtype);",
                               "n[e] = load(x, x_off + e, dtype) * r * load(w, d - 1 - e, dtype);"),
    "qknorm_rotate_before_norm_skipped": ("            rotate_half(n, k_rot + (t * hkv + h) * d, p, d, base);",
                                          "            for (int e = 0; e < d; ++e) k_rot[(t * hkv + h) * d + e] = n[e];"),
    "reglu_leaky": ("double relu = g > 0.0 ? g : 0.0;", "double relu = g > 0.0 ? g : 0.01 * g;"),
    "clip_gamma_from_alpha": ("double g = load(gamma, gamma_per_ch ? e : 0, dtype);",
                              "double g = load(alpha, alpha_per_ch ? e : 0, dtype);"),
    "clip_upper_bound_missing": ("                if (v > hi) v = hi;\n", ""),
    "clip_gamma_before_clamp": ("                double v = a * load(x, t * x_ts + h * x_hs + e, dtype);",
                                "                double v = a * g * load(x, t * x_ts + h * x_hs + e, dtype);"),
    "f16_bias_off_by_one": ("else mag = ldexp((double)(1024 + fr), ex - 25);",
                            "else mag = ldexp((double)(1024 + fr), ex - 24);"),
    "f16_no_subnormal_spacing": ("    if (lg < -14) lg = -14;\n    double q = ldexp(1.0, lg - 10);",
                                 "    double q = ldexp(1.0, lg - 10);"),
    "f16_truncates": ("double r = rint(a / q) * q;", "double r = floor(a / q) * q;"),
    "f16_overflow_at_max": ("if (a >= 65520.0) return", "if (a >= 65504.0) return"),
    "gqa_modulo": ("return h / (hq / hkv);", "return h % hkv;"),
    "add_norm_of_exact_sum": (
        "            store(x, r * x_stride + j, s, dtype);\n"
        "        }\n"
        "        rmsnorm_row(x, r * x_stride, w, y + r * y_stride, d, eps, dtype);",
        "            store(x, r * x_stride + j, s, dtype);\n"
        "            y[r * y_stride + j] = s;\n"
        "        }\n"
        "        {\n"
        "            double ss_ = 0.0;\n"
        "            for (int64_t j = 0; j < d; ++j) ss_ += y[r * y_stride + j] * y[r * y_stride + j];\n"
        "            for (int64_t j = 0; j < d; ++j)\n"
        "                y[r * y_stride + j] *= load(w, j, dtype) / sqrt(ss_ / (double)d + eps);\n"
        "        }"),
    "swiglu_sigmoid_of_up": ("double sigmoid = 1.0 / (1.0 + exp(-g));", "double sigmoid = 1.0 / (1.0 + exp(-u));"),
    "gather_reads_other_half": ("((((int64_t)which * num_blocks", "((((int64_t)(1 - which) * num_blocks"),
    "clip_lower_bound_missing": ("                if (v < lo) v = lo;\n", ""),
    "rope_position_off_by_one": ("int64_t p = positions[t];\n        for (int h = 0; h < hq; ++h)\n            rope_head(q",
                                 "int64_t p = positions[t] + 1;\n        for (int h = 0; h < hq; ++h)\n            rope_head(q"),
    "silu_missing_g": ("out[r * out_stride + c] = g * sigmoid * u;", "out[r * out_stride + c] = sigmoid * u;"),
    "clip_alpha_after_clamp": ("                double v = a * load(x, t * x_ts + h * x_hs + e, dtype);\n"
                               "                if (v < lo) v = lo;\n"
                               "                if (v > hi) v = hi;\n"
                               "                y[(t * n_head + h) * d + e] = v * g;",
                               "                double v = load(x, t * x_ts + h * x_hs + e, dtype);\n"
                               "                if (v < lo) v = lo;\n"
                               "                if (v > hi) v = hi;\n"
                               "                y[(t * n_head + h) * d + e] = a * v * g;"),
    "qknorm_mean_over_half": ("double r = 1.0 / sqrt(sum_sq / (double)d + eps);",
                              "double r = 1.0 / sqrt(sum_sq / (double)(d / 2) + eps);"),
    "scatter_offset_swapped": ("int64_t block = slot / block_size, offset = slot % block_size;",
                               "int64_t block = slot % block_size, offset = slot / block_size;"),
    "gather_offset_from_block": ("int64_t block = block_table[t / block_size], offset = t % block_size;",
                                 "int64_t block = block_table[t / block_size], offset = (t + 1) % block_size;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(oracle.SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = oracle.build(str(path), str(tmp_path / f"lib{name}.so"))
    L = oracle.lib(so)
    failed = []
    for pin, fn in PINS.items():
        try:
            fn(L)
        except AssertionError:
            failed.append(pin)
    assert failed, f"mutant {name} passed every pin"
