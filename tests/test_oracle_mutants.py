"""Planted mistakes in the oracle, on the CPU: every one must fail at least one pin.

Each mutant is a textual edit of a private copy of oracle.c (the real source is
never touched), compiled with gcc into a temporary directory. The edits are the
plausible slips: a wrong head-to-group map, a dropped scale, a sign error, a
missing normalisation, an off-by-one causal mask, wrong block or offset
arithmetic, a transposed operand, a wrong widening of stored values, a
window off by one, and in the quantised cache a wrong largest code, wrong
rounding, a wrong FP8 exponent bias or subnormal step, V scaled by K's scale,
signed codes read as unsigned, scales stored at the wrong slot, and for
per-channel scales the wrong KV head's or the K scales for V, transposed or
head-blind scale indexing, a subnormal scale taken as usable. All mutants
keep every memory access in bounds.
"""
from pathlib import Path

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTANTS = {
    "decode_group_map_mod": ("const int32_t g = h / group;                          /* [AE] 3.1",
                             "const int32_t g = h % n_kv;                          /* [AE] 3.1"),
    "prefill_group_map_mod": ("        const int32_t g = h / group;\n        const int32_t n_keys",
                              "        const int32_t g = h % n_kv;\n        const int32_t n_keys"),
    "dropped_scale": ("scores[t] = scale * dot - slope", "scores[t] = dot - slope"),
    "exp_sign_flip": ("const double w = exp(scores[t] - m);", "const double w = exp(m - scores[t]);"),
    "no_normalisation": ("out[c] /= den;", "out[c] /= 1.0;"),
    "den_squares": ("den += w;", "den += w * w;"),
    "causal_excludes_diagonal": ("causal ? i + 1 : seq_len", "causal ? (i > 0 ? i : 1) : seq_len"),
    "block_offset_shift": ("const int64_t off = t % block_size;",
                           "const int64_t off = (t + 1) % block_size;"),
    "block_index_halved": ("block_table[(int64_t)b * max_blocks_per_seq + t / block_size]",
                           "block_table[(int64_t)b * max_blocks_per_seq + t / block_size / 2]"),
    "block_row_of_next_sequence": (
        "block_table[(int64_t)b * max_blocks_per_seq + t / block_size]",
        "block_table[(int64_t)((b + 1) % batch) * max_blocks_per_seq + t / block_size]"),
    "append_offset_shift": ("const int64_t off = slot % block_size;\n        for (int32_t g = 0; g < n_kv; ++g) {\n            const size_t src",
                            "const int64_t off = (slot + 1) % block_size;\n        for (int32_t g = 0; g < n_kv; ++g) {\n            const size_t src"),
    "append_head_offset_transposed": (
        "const size_t dst = (((size_t)blk * n_kv + g) * block_size + off) * row;",
        "const size_t dst = (((size_t)blk * block_size + off) * n_kv + g) * row;"),
    "query_index_transposed": ("load_elem(q, q_dtype, ((int64_t)b * n_q + h) * head_dim + c)",
                               "load_elem(q, q_dtype, ((int64_t)h * batch + b) * head_dim + c)"),
    "values_read_from_keys": ("out[c] += w * key_elem(keys, 1, t, c, d)",
                              "out[c] += w * key_elem(keys, 0, t, c, d)"),
    "bf16_widening_shift": ("((uint32_t)h) << 16", "((uint32_t)h) << 15"),
    "f16_exponent_bias": ("ldexp((double)(1024 + frac), e - 25)",
                          "ldexp((double)(1024 + frac), e - 24)"),
    "max_tracks_minimum": ("if (scores[t] > m) m = scores[t];", "if (scores[t] < m) m = scores[t];"),
    "fp8_qmax_of_the_fnuz_format": ("fmt == ORACLE_FP8E4M3 ? 448.0f : 127.0f",
                                    "fmt == ORACLE_FP8E4M3 ? 240.0f : 127.0f"),
    "int8_truncates": ("fmaxf(rintf(y), -127.0f)", "fmaxf(truncf(y), -127.0f)"),
    "fp8_exponent_bias": ("ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 11)"),
    "fp8_encode_ties_away": ("double q = nearbyint((2.0 * fr - 1.0) * 8.0);",
                             "double q = round((2.0 * fr - 1.0) * 8.0);"),
    "fp8_subnormal_step": ("return sign | (uint8_t)nearbyint(ldexp(a, 9));",
                           "return sign | (uint8_t)nearbyint(ldexp(a, 8));"),
    "v_scaled_by_k_scale": ("const float* sc = is_v ? keys->v_scale : keys->k_scale;",
                            "const float* sc = is_v ? keys->k_scale : keys->k_scale;"),
    "int8_read_unsigned": ("case ORACLE_INT8: return (double)((const int8_t*)base)[idx];",
                           "case ORACLE_INT8: return (double)((const uint8_t*)base)[idx];"),
    "quant_append_scale_row_offset": ("const int64_t dst_row = (blk * n_kv + g) * block_size + off;",
                                      "const int64_t dst_row = (blk * n_kv + g) * block_size + (off + 1) % block_size;"),
    "channel_scales_of_kv_head_zero": ("keys.k_chan = k_scale + (int64_t)g * head_dim;",
                                       "keys.k_chan = k_scale;"),
    "channel_v_scaled_by_k_channels": ("const float* ch = is_v ? keys->v_chan : keys->k_chan;",
                                       "const float* ch = is_v ? keys->k_chan : keys->k_chan;"),
    "channel_append_scales_transposed": ("const int64_t sc = (int64_t)g * head_dim + c;",
                                         "const int64_t sc = (int64_t)c * n_kv + g;"),
    "channel_quantise_ignores_head": ("scales[(int64_t)g * d + c], fmt);", "scales[c], fmt);"),
    "channel_subnormal_scale_kept": ("if (!(s >= 0x1p-126f)) return 0;", "if (!(s > 0.0f)) return 0;"),
    "decode_window_one_too_wide": ("(window > 0 && ctx > window) ? ctx - window : 0",
                                   "(window > 0 && ctx > window) ? ctx - window - 1 : 0"),
    "prefill_window_one_too_narrow": ("(window > 0 && i + 1 > window) ? i + 1 - window : 0",
                                      "(window > 0 && i + 1 > window) ? i + 2 - window : 0"),
    "alibi_bias_sign": ("scale * dot - slope * (double)(qpos - (keys->kpos0 + t))",
                        "scale * dot + slope * (double)(qpos - (keys->kpos0 + t))"),
    "alibi_physical_key_position": ("slope * (double)(qpos - (keys->kpos0 + t))",
                                    "slope * (double)(qpos - keys->key_off[t] / d)"),
    "alibi_slope_of_the_kv_group": (
        "const double slope = alibi_slopes ? (double)alibi_slopes[h] : 0.0;\n            attend(qv, head_dim, scale, slope, (int64_t)ctx - 1",
        "const double slope = alibi_slopes ? (double)alibi_slopes[g] : 0.0;\n            attend(qv, head_dim, scale, slope, (int64_t)ctx - 1"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = oracle.SOURCE.read_text()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutant_src = tmp_path / "oracle_mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib = oracle.compile_library(mutant_src, tmp_path / "liboracle_mutant.so")
    orc = oracle.Oracle(lib)
    caught = []
    for pin_name, pin in ALL_PINS.items():
        try:
            pin(orc)
        except Exception as e:  # AssertionError, or a rejection the real oracle never raises
            caught.append((pin_name, type(e).__name__))
    assert caught, f"no pin catches mutant {name}"
