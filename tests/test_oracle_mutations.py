"""Plausible mistakes planted in copies of the CPU oracle (on the CPU) must be caught by the pins.

Each mutant is the oracle source with one text substitution (a dropped term, a wrong sign,
index, bound or rounding), compiled with gcc into a temporary directory and run through the pin
battery.  The unmodified oracle must pass the same battery.
"""
import os

import pytest

import oracle
from tests import pin_battery

MUTATIONS = {
    "scale_divisor": ("float s32 = a / (float)qmax;", "float s32 = a / (float)(qmax + 1);"),
    "truncate_not_round": ("float c = nearbyintf(y);", "float c = truncf(y);"),
    "no_clamp": ("if (c > (float)qmax) c = (float)qmax;", ""),
    "unrounded_scale": ("return (float)kvq_oracle_fp16_to_double(sb);", "return s32;"),
    "fp16_ties_away": ("double n = nearbyint(a / quantum);", "double n = round(a / quantum);"),
    "fp16_subnormal_floor": ("if (e < -14) e = -14;", "if (e < -15) e = -15;"),
    "v_group_stride": ("vrow + 32 * j", "vrow + 16 * j"),
    "v_nibble_unsigned": ("(int8_t)(nib >= 8 ? nib - 16 : nib)", "(int8_t)(nib)"),
    "k_scale_dropped": ("kd[d] = kcode * sk;", "kd[d] = kcode;"),
    "v_scale_group": ("kvq_oracle_fp16_to_double(vs[d / 32])", "kvq_oracle_fp16_to_double(vs[d / 64])"),
    "mask_off_by_one": ("*last = L - R + i;", "*last = L - R + i - 1;"),
    # fp8 (OCP E4M3 codes)
    "f8_fnuz_max": ("float s = group_scale(x, n, 448, scale_bits);",
                    "float s = group_scale(x, n, 240, scale_bits);"),
    "f8_bias_8": ("ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 11)"),
    "f8_subnormal_step": ("ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    "f8_ties_away": ("double r = nearbyint(a / quantum) * quantum;",
                     "double r = round(a / quantum) * quantum;"),
    "f8_zero_sign": ("uint8_t sign = signbit(y) ? 0x80 : 0;", "uint8_t sign = y < 0 ? 0x80 : 0;"),
    # sliding window over ring pages
    "window_off_by_one": ("*first = window > 0 ? *last - window + 1 : 0;",
                          "*first = window > 0 ? *last - window : 0;"),
    "window_from_row0": ("*first = window > 0 ? *last - window + 1 : 0;",
                         "*first = window > 0 ? L - R - window + 1 : 0;"),
    "ring_ignored": ("pt_row[ring > 0 ? (t / P) % ring : t / P]", "pt_row[t / P]"),
    "gqa_map_logits": ("int h = hq / G;", "int h = hq % Hkv;"),
    "gqa_map_values": ("int h = hq / (Hq / Hkv);", "int h = hq % Hkv;"),
    "exp_sign": ("w[t] = exp(w[t] - m);", "w[t] = exp(m - w[t]);"),
    "lse_drops_max": ("lse[o] = m + log(sum);", "lse[o] = log(sum);"),
    "default_scale": ("if (scale <= 0.0) scale = 1.0 / sqrt((double)D);\n  int count",
                      "if (scale <= 0.0) scale = 1.0 / (double)D;\n  int count"),
    "wrong_slot": ("kvq_oracle_read_slot_fmt(pool, P, Hkv, D, vb, page, t % P, h, kc, &ks, vc, vs);",
                   "kvq_oracle_read_slot_fmt(pool, P, Hkv, D, vb, page, (t + 1) % P, h, kc, &ks, vc, vs);"),
    "k_tokens_swapped": ("(size_t)16 * t + (size_t)(d % 16)", "(size_t)16 * (t ^ 1) + (size_t)(d % 16)"),
    "v_lane_transposed": ("int lane = 16 * (t / 4) + d % 16;\n  int r = t % 4;",
                          "int lane = 16 * (t % 4) + d % 16;\n  int r = t / 4;"),
    "wrong_query_row": ("q + (((size_t)b * R + i) * Hq + hq) * D",
                        "q + (((size_t)b * R + (R - 1)) * Hq + hq) * D"),
    "no_normalize": ("for (int t = first; t <= last; ++t) w[t] /= sum;", ""),
    "no_running_max": ("if (w[t] > m) m = w[t];", "m = 0.0;"),
    # page-table entries outside the pool (clamped into [0, num_pages))
    "page_clamp_low_wraps": ("if (page < 0) page = 0;", "if (page < 0) page = num_pages - 1;"),
    "page_clamp_high_to_zero": ("if (page >= num_pages) page = num_pages - 1;",
                                "if (page >= num_pages) page = 0;"),
    # K8/V8 (8-bit V codes)
    "v8_qmax": ("const int vqmax = vb == 8 ? 127 : 7;", "const int vqmax = vb == 8 ? 63 : 7;"),
    "v8_dim_pair_bit": ("(size_t)4 * ((d / 16) % 2) + (size_t)(t % 4)",
                        "(size_t)4 * ((d / 32) % 2) + (size_t)(t % 4)"),
    "v8_scale_section": ("(size_t)P * D * vb / 8 + (size_t)2 * ((size_t)s * (D / 32) + j)",
                         "(size_t)P * D / 2 + (size_t)2 * ((size_t)s * (D / 32) + j)"),
}


def test_unmodified_oracle_passes_the_battery():
    assert pin_battery.run(oracle.default()) == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique or missing"
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.build(force=True, source=path, out=os.path.join(tmp_path, "libmutant.so"))
    failed = pin_battery.run(oracle.Oracle(lib))
    assert failed, f"mutation {name} slipped past every pin"
