"""The pins are strong enough: each plausible mistake planted in a copy of the
oracle's C source (on the CPU, in a temporary directory) makes at least one
pin fail. The real oracle file is never modified."""
import os

import pytest

import oracle as O
from oracle_pins import PINS

SRC = os.path.join(os.path.dirname(O.__file__), "gqa_oracle.c")

# (name, exact text in the oracle, replacement)
MUTANTS = [
    ("group_floor_plus_one", "int64_t g1 = (num + H - 1) / H;", "int64_t g1 = num / H + 1;"),
    ("group_off_by_one", "return (int)(g1 - 1);", "return (int)(g1 % G);"),
    ("dropped_scale", "s[t] = scale * dot;", "s[t] = dot;"),
    ("exp_sign", "s[t] = exp(s[t] - m);", "s[t] = exp(m - s[t]);"),
    ("no_normalise", "out[d] = acc / denom;", "out[d] = acc;"),
    ("keys_from_values", "dot += widen(q, q_off + d, dtype) * widen(k,", "dot += widen(q, q_off + d, dtype) * widen(v,"),
    ("head_major_cache", "int64_t key_stride = (int64_t)G * D; ", "int64_t key_stride = (int64_t)D; "),
    ("causal_drops_diagonal", "int L = causal ? t + 1 : T;", "int L = causal ? t : T;"),
    ("causal_ignored", "int L = causal ? t + 1 : T;", "int L = T;"),
    ("prefill_scale_dh", "double scale = 1.0 / sqrt((double)D);", "double scale = 1.0 / (double)D;"),
    ("pool_divides_by_H", "o[d] = o[d] / (double)members;", "o[d] = o[d] / (double)H;"),
    ("cache_single_tensor", "return 2.0 * (double)kv_heads", "return 1.0 * (double)kv_heads"),
    ("clamp_off_by_one", "if (L > Tmax)\n        return Tmax;", "if (L > Tmax)\n        return Tmax - 1;"),
    ("bf16_low_half", "<< 16;\n        float f;", ";\n        float f;"),
    ("prefill_wrong_group", "int g = oracle_group_of_head(h, H, G);\n        int L = causal",
     "int g = h % G;\n        int L = causal"),
    ("f16_exponent_bias", "mag = ldexp((double)(frac + 1024), ex - 25);", "mag = ldexp((double)(frac + 1024), ex - 24);"),
    ("f16_subnormal_scale", "mag = ldexp((double)frac, -24);", "mag = ldexp((double)frac, -25);"),
    ("append_overwrites_last", "size_t dst = ((size_t)b * Tmax + L) * row;",
     "size_t dst = ((size_t)b * Tmax + (L > 0 ? L - 1 : 0)) * row;"),
    ("append_not_attended", "            L = L + 1;\n", ""),
    ("window_one_short", "int lo = (window > 0 && L > window) ? L - window : 0;",
     "int lo = (window > 0 && L > window) ? L - window + 1 : 0;"),
    ("prefill_window_one_long", "int lo = (window > 0 && t + 1 > window) ? t + 1 - window : 0;",
     "int lo = (window > 0 && t + 1 > window) ? t - window : 0;"),
    ("prefill_window_scale", "double inv_sqrt_d = 1.0 / sqrt((double)D);", "double inv_sqrt_d = 1.0 / (double)D;"),
    ("weighted_pool_ignores_weights", "o[d] += w[i] * widen(in,", "o[d] += widen(in,"),
    ("window_one_long", "int lo = (window > 0 && L > window) ? L - window : 0;",
     "int lo = (window > 0 && L > window) ? L - window - 1 : 0;"),
    ("append_value_not_written", "            memcpy((char *)v + dst, (const char *)v_new + (size_t)b * row, row);\n", ""),
    ("no_max_subtraction", "s[t] = exp(s[t] - m);", "s[t] = exp(s[t]);"),
    ("max_of_first_key_only", "if (s[t] > m)\n            m = s[t];", "if (t == 0)\n            m = s[t];"),
    ("pool_strided_groups", "if (oracle_group_of_head(i, H, G) != g)\n                    continue;\n                ++members;",
     "if (i % G != g)\n                    continue;\n                ++members;"),
    ("values_from_keys", "acc += s[t] * widen(v, key_base", "acc += s[t] * widen(k, key_base"),
    ("decode_query_of_group", "attend_row(q, row * D, k, v, key_base, key_stride, L, D,",
     "attend_row(q, ((int64_t)b * H + g) * D, k, v, key_base, key_stride, L, D,"),
    ("prefill_window_one_short", "int lo = (window > 0 && t + 1 > window) ? t + 1 - window : 0;",
     "int lo = (window > 0 && t + 1 > window) ? t + 2 - window : 0;"),
    ("weighted_pool_group_weight", "o[d] += w[i] * widen(in,", "o[d] += w[g] * widen(in,"),
    ("f16_sign_dropped", "return sign ? -mag : mag;", "return mag;"),
    ("empty_row_not_zero", "if (L <= 0) {", "if (L < 0) {"),
    ("prefill_query_of_group",
     "int64_t q_off = (((int64_t)b * T + t) * H + h) * D;\n        int64_t key_base = ((int64_t)b * T * G + g) * D;",
     "int64_t q_off = (((int64_t)b * T + t) * H + g) * D;\n        int64_t key_base = ((int64_t)b * T * G + g) * D;"),
    ("prefill_keys_of_first_sequence", "int64_t key_base = ((int64_t)b * T * G + g) * D;",
     "int64_t key_base = ((int64_t)g) * D;"),
]


def _run_pins(lib):
    failed = []
    for pin in PINS:
        try:
            pin(lib)
        except Exception as e:  # any assertion or crash-free error counts as caught
            failed.append((pin.__name__, type(e).__name__))
    return failed


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    src = tmp_path / f"{name}.c"
    src.write_text(text.replace(old, new))
    so = O.build(str(src), str(tmp_path / f"{name}.so"))
    lib = O.load(so)
    failed = _run_pins(lib)
    assert failed, f"planted mistake {name} passed every pin"
