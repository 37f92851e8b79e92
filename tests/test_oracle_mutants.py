"""The oracle pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of the oracle's C source (a dropped
term, a wrong sign, index or bound, a transposed operand), builds it into a
temporary library, runs the pins of test_oracle.py against it and requires at
least one pin to fail.  The real oracle is never modified.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "sdpa_oracle.c")

MUTANTS = {
    "gqa_index_modulo": ("const int64_t g = h / group;", "const int64_t g = h % p->kv_heads;"),
    "causal_strict": ("j <= i + delta", "j < i + delta"),
    "default_offset_sign": ("p->k_len - p->q_len", "p->q_len - p->k_len"),
    "mask_dropped": ("sj += (double)mask", "sj -= 0.0 * (double)mask"),
    "mask_before_scale": ("double sj = scale * dot;", "double sj = dot;"),
    "default_scale": ("1.0 / sqrt((double)D)", "1.0 / (double)D"),
    "lse_sign": ("*lse_out = m + log(l);", "*lse_out = m - log(l);"),
    "policy_swapped": ("p->masked_zero ? 0.0 : NAN", "p->masked_zero ? NAN : 0.0"),
    "v_uses_k_strides": ("b * p->vs[0] + g * p->vs[1] + j * p->vs[2]",
                         "b * p->ks[0] + g * p->ks[1] + j * p->ks[2]"),
    "key_length_off_by_one": ("(j < kv_len)", "(j <= kv_len)"),
    "f16_exponent_bias": ("e - 25", "e - 24"),
    "bf16_wrong_half": ("(uint32_t)b << 16", "(uint32_t)b << 15"),
    "bad_row_ignored": ("            bad = 1;", "            bad = 0;"),
    "max_not_subtracted": ("l += exp(s[j] - m);", "l += exp(s[j]);"),
    "weights_not_normalised": ("exp(s[j] - m) / l;", "exp(s[j] - m);"),
    "q_row_stride_ignored": ("i * p->qs[2];", "0 * p->qs[2];"),
    "explicit_offset_ignored": ("p->has_offset == 1   ? p->causal_offset",
                                "0 ? p->causal_offset"),
    "end_offset_uses_capacity": ("p->has_offset == 2 ? kv_len - p->q_len",
                                 "p->has_offset == 2 ? p->k_len - p->q_len"),
    "end_offset_ignored": ("p->has_offset == 2 ? kv_len", "0 ? kv_len"),
    "window_strict": ("j >= i + delta - p->window", "j > i + delta - p->window"),
    "window_ignored": ("(p->window < 0 ||", "(1 ||"),
    "softcap_ignored": ("            sj = p->softcap * tanh(sj / p->softcap);\n",
                        "            sj = sj;\n"),
    "softcap_after_mask": (
        "        if (p->softcap > 0.0)\n            sj = p->softcap * tanh(sj / p->softcap);\n"
        "        if (mask)\n            sj += (double)mask[b * p->ms[0] + h * p->ms[1] + i * p->ms[2] + j];\n",
        "        if (mask)\n            sj += (double)mask[b * p->ms[0] + h * p->ms[1] + i * p->ms[2] + j];\n"
        "        if (p->softcap > 0.0)\n            sj = p->softcap * tanh(sj / p->softcap);\n"),
    "sink_not_in_denominator": ("double l = p->sink ? exp(sink - m) : 0.0;", "double l = 0.0;"),
    "sink_ignores_head": ("(double)head_sink[h]", "(double)head_sink[0]"),
    "channel_scale_ignores_head": ("scale[g * p->head_dim + d]", "scale[d]"),
    "channel_scale_transposed": ("scale[g * p->head_dim + d]", "scale[d * p->kv_heads + g]"),
    "v_uses_k_scale": ("load_kv(p, v, v_scale, p->v_quant", "load_kv(p, v, k_scale, p->k_quant"),
    "int8_unscaled": ("return x * (double)(quant == 1", "return x * 1.0 + 0.0 * (double)(quant == 1"),
    "doc_start_strict": ("j >= first_key", "j > first_key"),
    "doc_start_ignored": ("doc_start ? (int64_t)doc_start[b * p->q_len + i] : 0",
                          "doc_start ? 0 * (int64_t)doc_start[0] : 0"),
    "doc_start_wrong_row": ("doc_start[b * p->q_len + i]", "doc_start[b * p->q_len]"),
    "key_lengths_ignored": ("kv_len = L < 0 ? 0 : (L > p->k_len ? p->k_len : L);",
                            "kv_len = p->k_len; (void)L;"),
}

CHECKS = [
    pins.test_decode_f16_all_patterns,
    pins.test_decode_bf16_all_patterns,
    lambda: pins.test_weights_sum_to_one("f16"),
    pins.test_uniform_scores_give_mean_and_log_count,
    lambda: pins.test_one_hot_is_exact("bf16"),
    pins.test_two_keys_logistic,
    pins.test_default_scale_is_inverse_sqrt_head_dim,
    pins.test_gqa_mapping_golden,
    pins.test_causal_visible_counts_golden,
    pins.test_default_offset_is_klen_minus_qlen,
    pins.test_negative_offset_empties_leading_rows,
    pins.test_end_aligned_visible_counts_golden,
    pins.test_end_aligned_equals_sliced_cache,
    pins.test_window_visible_counts_golden,
    pins.test_sink_closed_form_uniform_scores,
    pins.test_sink_row_without_keys_is_zero_under_both_policies,
    pins.test_softcap_two_keys_logistic,
    pins.test_softcap_comes_before_the_mask,
    pins.test_key_length_zero_and_beyond_capacity,
    pins.test_hidden_keys_are_never_read,
    pins.test_mask_hidden_keys_weigh_zero,
    pins.test_layouts_and_broadcast_agree,
] + [(lambda r=r: pins.test_special_values_golden(r)) for r in pins._golden("special_values.txt")] \
  + [(lambda c=c: pins.test_brute_force_against_library_route(c, "nan")) for c in pins.BRUTE] \
  + [(lambda c=c: pins.test_variants_against_library_route(c, "nan"))
     for c in pins.BRUTE_VARIANTS] \
  + [lambda: pins.test_int8_cache_equals_exact_float_cache(True),
     lambda: pins.test_int8_cache_equals_exact_float_cache(False)] \
  + [(lambda c=c: pins.test_int8_cache_against_library_route(c)) for c in pins.INT8_CASES] \
  + [pins.test_doc_mask_visible_counts_golden, pins.test_doc_mask_equals_separate_documents] \
  + [(lambda c=c: pins.test_doc_mask_against_library_route(c)) for c in pins.DOC_CASES]


def _any_check_fails():
    for check in CHECKS:
        try:
            check()
        except (AssertionError, RuntimeError, ValueError):
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor not found: %r" % old
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib_path = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           "-o", str(lib_path), str(mutated), "-lm"])
    real = oracle._load()
    lib = ctypes.CDLL(str(lib_path))
    for fn in ("oracle_attention", "oracle_decode_f16", "oracle_decode_bf16"):
        getattr(lib, fn).restype = getattr(real, fn).restype
        getattr(lib, fn).argtypes = getattr(real, fn).argtypes
    monkeypatch.setattr(oracle, "_lib", lib)
    assert _any_check_fails(), "no pin caught mutant %s" % name


def test_unmutated_oracle_passes_every_check():
    assert not _any_check_fails()
