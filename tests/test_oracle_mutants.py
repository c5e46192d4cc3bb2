"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant is a copy of oracle/q4_oracle.c with one plausible slip (a wrong
rounding, sign, index, clamp, nibble order, divisor ...), built with the same
flags into a temporary directory.  Everything happens on the CPU.
"""
import os

import pytest

import oracle
from oracle import build as obuild
from pins import (ALL_PINS, pin_brute_force_int8_per_channel, pin_kv_brute_force,
                  pin_w8a8_row_quantizers)

# the pins that take seconds run last, so most mutants are caught cheaply
_SLOW = (pin_brute_force_int8_per_channel, pin_kv_brute_force, pin_w8a8_row_quantizers)
_CHEAP_FIRST = [p for p in ALL_PINS if p not in _SLOW] + list(_SLOW)

MUTANTS = {
    "round_half_up": ("rintf(v[i] / s) + (float)z", "floorf(v[i] / s + 0.5f) + (float)z"),
    "zero_point_sign": ("rintf(-mn / s)", "rintf(mn / s)"),
    "zero_point_unclipped": ("(int32_t)clampf(rintf(-mn / s), 0.0f, qmax)",
                             "(int32_t)rintf(-mn / s)"),
    "no_scale_floor_asym": ("        float s = (mx - mn) / qmax;\n        if (s < 1e-8f) s = 1e-8f;",
                            "        float s = (mx - mn) / qmax;"),
    "asym_divisor_2b": ("float s = (mx - mn) / qmax;", "float s = (mx - mn) / (qmax + 1.0f);"),
    "sym_divisor_2b_minus_1": ("const float qmax = (float)((1 << (bits - 1)) - 1);",
                               "const float qmax = (float)((1 << bits) - 1);"),
    "sym_offset_7": ("codes[t] + offset : codes[t]", "codes[t] + offset - 1 : codes[t]"),
    "sym_offset_fixed_8": ("const int64_t groups = n_in / group_size;\n    const int32_t offset = 1 << (bits - 1);",
                           "const int64_t groups = n_in / group_size;\n    const int32_t offset = 8;"),
    "nibble_order_reversed": ("row[k / per_word] |= u << (bits * (k % per_word));",
                              "row[k / per_word] |= u << (bits * (per_word - 1 - k % per_word));"),
    "pack_shift_4": ("row[k / per_word] |= u << (bits * (k % per_word));",
                     "row[k / per_word] |= u << (4 * (k % per_word));"),
    "group_capped_1024": ("orc_quantize_group(v, group_size, bits, symmetric, &s, &z, codes);",
                          "orc_quantize_group(v, group_size > 1024 ? 1024 : group_size, bits, symmetric, &s, &z, codes);"),
    "min_init_zero": ("float mn = v[0], mx = v[0];", "float mn = 0.0f, mx = v[0];"),
    "dequant_sign": ("out[n * n_in + k] = s * (float)(u - z);",
                     "out[n * n_in + k] = s * (float)(z - u);"),
    "dequant_group_index": ("float s = orc_f16_to_f32(scales[n * groups + k / group_size]);",
                            "float s = orc_f16_to_f32(scales[n * groups + (k / group_size + 1) % groups]);"),
    "dequant_nibble_index": ("int32_t u = (int32_t)((word >> (bits * (k % per_word))) & mask);",
                             "int32_t u = (int32_t)((word >> (bits * ((k + 1) % per_word))) & mask);"),
    "dequant_mask_4bit": ("const uint32_t mask = (1u << bits) - 1u;", "const uint32_t mask = 0xFu;"),
    "f16_truncate": ("if (rem > half || (rem == half && (q & 1u)))", "if (0)"),
    "f16_ties_away": ("if (rem > half || (rem == half && (q & 1u)))", "if (rem >= half)"),
    "f16_subnormal_scale": ("float mag = (float)frac * 0x1p-24f;", "float mag = (float)frac * 0x1p-23f;"),
    "linear_reversed_k": ("(double)orc_f16_to_f32(x_f16[i * n_in + k])",
                          "(double)orc_f16_to_f32(x_f16[i * n_in + (n_in - 1 - k)])"),
    "linear_abs_dropped": ("acc_abs += fabs(p);", "acc_abs += p;"),
    "linear_row_swap": ("y[i * n_out + n] = acc;", "y[i * n_out + (n_out - 1 - n)] = acc;"),
    "kv_channel_stride": ("v[i] = orc_f16_to_f32(xb[(int64_t)i * d + j]);",
                          "v[i] = orc_f16_to_f32(xb[(int64_t)j * t + i]);"),
    "kv_channel_scale_index": ("scale[b * d + j] = s;", "scale[b * d + (d - 1 - j)] = s;"),
    "kv_token_asymmetric": ("orc_quantize_group(v, d, bits, 1, &s, &z, c);",
                            "orc_quantize_group(v, d, bits, 0, &s, &z, c);"),
    "kv_dequant_channel_scale": ("out[e] = orc_f32_to_f16((float)q[e] * scale[b * d + j]);",
                                 "out[e] = orc_f32_to_f16((float)q[e] * scale[b * d + i % d]);"),
    "kv_dequant_double_f16": ("out[r * d + i] = orc_f32_to_f16((float)q[r * d + i] * scale[r]);",
                              "out[r * d + i] = orc_f32_to_f16((float)q[r * d + i] * orc_f16_to_f32(orc_f32_to_f16(scale[r])));"),
    "kv_cache_bytes_one_side": ("return 2.0 * (double)layers", "return 1.0 * (double)layers"),
    "sq_ratio_inverted": ("float v = num / den;", "float v = den / num;"),
    "sq_pow_exponents_swapped": ("num = powf(act_max[j], alpha);\n            den = powf(w, 1.0f - alpha);",
                                 "num = powf(act_max[j], 1.0f - alpha);\n            den = powf(w, alpha);"),
    "sq_no_weight_floor": ("const float w = w_max[j] < 1e-5f ? 1e-5f : w_max[j];", "const float w = w_max[j];"),
    "sq_colmax_no_abs": ("const float a = fabsf(orc_f16_to_f32(x[r * cols + j]));",
                         "const float a = orc_f16_to_f32(x[r * cols + j]);"),
    "w8a8_act_multiplied": ("v[j] = s ? xv / s[j] : xv;", "v[j] = s ? xv * s[j] : xv;"),
    "w8a8_weight_divided": ("v[k] = s ? w[n * n_in + k] * s[k] : w[n * n_in + k];",
                            "v[k] = s ? w[n * n_in + k] / s[k] : w[n * n_in + k];"),
    "w8a8_epilogue_scale_swap": ("const float v = ((float)a * sx[i]) * sw[n];",
                                 "const float v = ((float)a * sw[n]) * sw[n];"),
    "w8a8_gemm_k_shift": ("a += (int64_t)qx[i * k + j] * (int64_t)qw[n * k + j];",
                          "a += (int64_t)qx[i * k + j] * (int64_t)qw[n * k + (j + 1) % k];"),
    "gptq_hessian_not_doubled": ("            h[i * n + j] = 2.0 * acc;\n            h[j * n + i] = 2.0 * acc;",
                                 "            h[i * n + j] = acc;\n            h[j * n + i] = acc;"),
    "gptq_damp_sum_not_mean": ("const double add = lambda * (sum / (double)n);", "const double add = lambda * sum;"),
    "gptq_factor_not_reversed": ("a[i * n + k] = h[(n - 1 - i) * n + (n - 1 - k)];", "a[i * n + k] = h[i * n + k];"),
    "gptq_error_undivided": ("const float err = (row[i] - deq) / u[i * n + i];", "const float err = row[i] - deq;"),
    "gptq_update_sign": ("row[j] = row[j] - err * u[i * n + j];", "row[j] = row[j] + err * u[i * n + j];"),
    "gptq_error_fp32_scale": ("const float deq = s16 * (q - (float)z);", "const float deq = s * (q - (float)z) * 1.001f;"),
    "awq_mean_signed": ("acc += fabs((double)orc_f16_to_f32(x[r * n + j]));", "acc += (double)orc_f16_to_f32(x[r * n + j]);"),
    "awq_alpha_complement": ("const float v = (float)pow(mean[j], alpha);", "const float v = (float)pow(mean[j], 1.0 - alpha);"),
    "awq_eff_multiplied": ("w_eff[r * n + k] = ws[r * n + k] / s[k];", "w_eff[r * n + k] = ws[r * n + k] * s[k];"),
    "awq_loss_unsquared": ("acc += y * y;", "acc += fabs(y);"),
}


def _failing_pins(orc, first_only=False):
    failed = []
    for pin in _CHEAP_FIRST:
        try:
            pin(orc, quick=True)
        except AssertionError:
            failed.append(pin.__name__)
            if first_only:
                break
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(obuild.SRC, encoding="utf-8").read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique in the oracle source"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new), encoding="utf-8")
    lib = obuild.build(str(path), str(tmp_path / f"lib_{name}.so"), extra_flags=["-w"])
    failed = _failing_pins(oracle.Oracle(lib), first_only=True)
    assert failed, f"mutant {name} passes every pin"


def test_unmutated_copy_passes_quick_pins(tmp_path):
    lib = obuild.build(obuild.SRC, str(tmp_path / "lib_copy.so"))
    assert _failing_pins(oracle.Oracle(lib)) == []
    assert os.path.exists(lib)
