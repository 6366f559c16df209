"""Mutation check of the oracle's pins (CPU only).

Each mutant is a copy of oracle.c with one plausible slip planted in it; it is
compiled to a temporary library and the pins of ``test_oracle_pins`` are run
against it.  Every mutant must fail at least one pin -- otherwise the pins
would not be able to tell that slip from the correct oracle.
"""
import os
import subprocess
import sys

import pytest

import oracle

SRC = open(oracle.SOURCE).read()

MUTANTS = {
    "gqa_h_mod_G": ("const int g = h / G;", "const int g = h % G;"),
    "block_index_mod": ("block_tables[(int64_t)s * MB + t / BS]", "block_tables[(int64_t)s * MB + t % BS]"),
    "slot_index_div": ("int r = t % BS;", "int r = t / BS;"),
    "no_scale": ("scores[t] = sc * dot;", "scores[t] = dot;"),
    "sign_of_dot": ("dot += qd[i] *", "dot -= qd[i] *"),
    "k_used_as_v": ("o[i] += e * kv_elem(src, 1,", "o[i] += e * kv_elem(src, 0,"),
    "v_used_as_k": ("dot += qd[i] * kv_elem(src, 0,", "dot += qd[i] * kv_elem(src, 1,"),
    "no_normalisation": ("for (int i = 0; i < D; ++i) o[i] /= denom;", ""),
    "one_token_short": ("for (int t = 0; t < n; ++t) {\n            int64_t b", "for (int t = 0; t < n - 1; ++t) {\n            int64_t b"),
    "head_major_slot": ("int64_t slot = (b * BS + r) * (int64_t)Hkv + g;",
                        "int64_t slot = (b * Hkv + g) * (int64_t)BS + r;"),
    "int8_no_dequant": ("return (double)base[slot * D + i] * (double)sc[slot];",
                        "return (double)base[slot * D + i];"),
    "int8_k_scales_for_v": ("const float *sc = which_v ? src->v_scales : src->k_scales;",
                            "const float *sc = src->k_scales;"),
    "quant_divisor_128": ("float s = amax / 127.0f;", "float s = amax / 128.0f;"),
    "quant_truncates": ("nearbyintf(xr[i] / s)", "truncf(xr[i] / s)"),
    "max_not_subtracted_in_exp": ("double e = exp(scores[t] - m);", "double e = exp(scores[t] - 2.0 * m);"),
    "write_block_mod": ("const int64_t block = slots[t] / BS;", "const int64_t block = slots[t] % BS;"),
    "write_offset_div": ("const int64_t offset = slots[t] % BS;", "const int64_t offset = slots[t] / BS;"),
    "write_key_into_v": ("v_cache[dst + i] = value[", "v_cache[dst + i] = key["),
    "write_head_major": ("const int64_t dst = ((block * BS + offset) * Hkv + g) * (int64_t)D;",
                         "const int64_t dst = ((block * Hkv + g) * BS + offset) * (int64_t)D;"),
    "write_head_ignored": ("k_cache[dst + i] = key[t * key_stride + (int64_t)g * D + i];",
                           "k_cache[dst + i] = key[t * key_stride + i];"),
    "int8_write_cell_ignores_head": ("const int64_t cell = (block * BS + offset) * Hkv + g;",
                                     "const int64_t cell = (block * BS + offset) * Hkv;"),
    "int8_write_v_from_key": ("row[i] = (float)bf16_bits_to_double(value[",
                              "row[i] = (float)bf16_bits_to_double(key["),
    "int8_write_v_scale_into_k": ("v_cache + cell * D, v_scales + cell);",
                                  "v_cache + cell * D, k_scales + cell);"),
    "fp8_exponent_bias_8": ("v = ldexp(1.0 + m / 8.0, e - 7);", "v = ldexp(1.0 + m / 8.0, e - 8);"),
    "fp8_subnormal_as_normal": ("v = ldexp((double)m, -9);", "v = ldexp(1.0 + m / 8.0, -7);"),
    "fp8_ties_to_odd": ("(d == best_d && (c & 1) == 0)", "(d == best_d && (c & 1) == 1)"),
    "fp8_saturates": ("if (a > 464.0) return (uint8_t)(sign | 0x7F);",
                      "if (a > 464.0) return (uint8_t)(sign | 0x7E);"),
    "fp8_nan_loses_sign": ("if (isnan(x) || isinf(x)) return (uint8_t)(sign | 0x7F);",
                           "if (isnan(x) || isinf(x)) return (uint8_t)0x7F;"),
    "fp8_cache_read_as_integers": ("return oracle_fp8_e4m3_to_double(base[slot * D + i]);",
                                   "return (double)base[slot * D + i];"),
    "fp8_write_value_from_key": ("v_cache[dst + i] = oracle_fp8_e4m3_from_double(\n                    bf16_bits_to_double(value[",
                                 "v_cache[dst + i] = oracle_fp8_e4m3_from_double(\n                    bf16_bits_to_double(key["),
    "score_ratio_inverted": ("scores[b * BS + r] = sqrt(vv) / sqrt(kk);",
                             "scores[b * BS + r] = sqrt(kk) / sqrt(vv);"),
    "score_without_sqrt": ("scores[b * BS + r] = sqrt(vv) / sqrt(kk);", "scores[b * BS + r] = vv / kk;"),
    "score_at_logical_position": ("scores[b * BS + r] = sqrt(vv) / sqrt(kk);",
                                  "scores[(int64_t)s * MB * BS + t] = sqrt(vv) / sqrt(kk);"),
    "evict_mean_of_logical_slots": ("const float *blk = scores + (int64_t)row[j] * BS;",
                                    "const float *blk = scores + (int64_t)j * BS;"),
    "score_first_head_only": ("double kk = 0.0, vv = 0.0;\n            for (int g = 0; g < Hkv; ++g) {",
                              "double kk = 0.0, vv = 0.0;\n            for (int g = 0; g < 1; ++g) {"),
    "score_ignores_begin": ("for (int t = token_begin ? token_begin[s] : 0; t < n; ++t) {",
                            "for (int t = 0; t < n; ++t) {"),
    "evict_argmax": ("if (victim < 0 || mean < best) {", "if (victim < 0 || mean > best) {"),
    "evict_ties_to_last": ("if (victim < 0 || mean < best) {", "if (victim < 0 || mean <= best) {"),
    "evict_nan_candidate": ("            if (isnan(mean)) continue;\n", ""),
    "evict_partial_block_candidate": ("const int n_full = n / BS;", "const int n_full = (n + BS - 1) / BS;"),
    "evict_table_not_shifted": ("for (int j = victim; j + 1 < nblk; ++j) row[j] = row[j + 1];",
                                "for (int j = victim + 1; j + 1 < nblk; ++j) row[j] = row[j + 1];"),
    "evict_context_kept": ("context_lens[s] = n - BS;", "context_lens[s] = n;"),
    "prefill_position_from_chunk_start": ("const int p = context_lens[s] - nq + i;", "const int p = i;"),
    "prefill_excludes_itself": ("block_tables + (int64_t)s * MB, p + 1, h / G,",
                                "block_tables + (int64_t)s * MB, p, h / G,"),
    "prefill_head_mod": ("block_tables + (int64_t)s * MB, p + 1, h / G,",
                         "block_tables + (int64_t)s * MB, p + 1, h % Hkv,"),
    "prefill_int8_scales_swapped": ("kv_src src = {KV_INT8, k_cache, v_cache, k_scales, v_scales};\n    return prefill_common",
                                    "kv_src src = {KV_INT8, k_cache, v_cache, v_scales, k_scales};\n    return prefill_common"),
    "prefill_fp8_caches_swapped": ("kv_src src = {KV_FP8, k_cache, v_cache, NULL, NULL};\n    return prefill_common",
                                   "kv_src src = {KV_FP8, v_cache, k_cache, NULL, NULL};\n    return prefill_common"),
    "prefill_k_as_v": ("const double e = exp(scores[t] - m);\n        denom += e;\n        for (int i = 0; i < D; ++i) o[i] += e * kv_elem(src, 1,",
                       "const double e = exp(scores[t] - m);\n        denom += e;\n        for (int i = 0; i < D; ++i) o[i] += e * kv_elem(src, 0,"),
    "compress_keeps_lowest": ("if (!an && a->score != b->score) return a->score > b->score ? -1 : 1;",
                              "if (!an && a->score != b->score) return a->score > b->score ? 1 : -1;"),
    "compress_ties_keep_later": ("return (a->pos > b->pos) - (a->pos < b->pos);     /* then earlier first */",
                                 "return (a->pos < b->pos) - (a->pos > b->pos);"),
    "compress_nan_ranks_last": ("if (an != bn) return an ? -1 : 1;", "if (an != bn) return an ? 1 : -1;"),
    "compress_kept_in_rank_order": ("qsort(keep, (size_t)budget, sizeof *keep, int_cmp);", ""),
    "compress_scores_stay": ("            scores[slot] = f[2 * ns];\n", ""),
    "compress_v_from_k": ("memcpy(vb + (size_t)j * row_bytes, v_cache + slot", "memcpy(vb + (size_t)j * row_bytes, k_cache + slot"),
    "compress_context_kept": ("        context_lens[s] = budget;\n", ""),
    "compress_k_scales_stay": ("                k_scales[slot * Hkv + g] = f[g];\n", ""),
    "compress_one_kept_short": ("for (int j = 0; j < budget; ++j) keep[j] = rk[j].pos;",
                                "for (int j = 0; j < budget; ++j) keep[j] = rk[j > 0 ? j - 1 : 0].pos;"),
}

PIN_FUNCS = [
    "test_context_one_returns_v_exactly",
    "test_context_zero_gives_zero_row",
    "test_gqa_groups_are_consecutive_heads",
    "test_scale_zero_gives_mean_over_exactly_the_valid_tokens",
    "test_two_tokens_closed_form_logistic",
    "test_uniform_keys_give_mean_of_values",
    "test_tiny_workload_matches_sdpa",
    "test_int8_matches_sdpa_on_dequantized_cache",
    "test_quantizer_closed_form_properties",
    "test_int8_matches_bf16_on_lossless_values",
    "test_generator_int8_synthesis_matches_oracle_quantizer",
    "test_write_then_decode_matches_sdpa_on_appended_context",
    "test_write_places_rows_at_flat_slot_and_leaves_the_rest",
    "test_write_rejects_out_of_range_and_duplicate_slots",
    "test_int8_write_of_lossless_rows_is_exact_per_head",
    "test_int8_write_error_bound_and_decode_against_dequantized_sdpa",
    "test_fp8_decode_of_every_code_matches_torch",
    "test_fp8_cast_of_every_bf16_matches_torch",
    "test_fp8_decode_matches_sdpa_on_decoded_cache",
    "test_fp8_matches_bf16_on_the_same_values",
    "test_fp8_write_then_decode_matches_sdpa_on_appended_context",
    "test_token_scores_closed_form_on_constant_rows",
    "test_token_scores_match_norms_all_kinds",
    "test_token_scores_scale_with_v_and_inversely_with_k",
    "test_evict_removes_the_lowest_mean_full_block",
    "test_evict_ties_take_the_lowest_block_and_nan_is_never_chosen",
    "test_evict_masked_and_short_sequences_are_untouched",
    "test_decode_after_eviction_equals_attention_without_the_block",
    "test_prefill_single_query_is_the_decode",
    "test_prefill_whole_prompt_matches_causal_sdpa",
    "test_prefill_chunk_after_a_cached_prefix_matches_masked_sdpa",
    "test_prefill_is_causal",
    "test_prefill_int8_single_query_is_the_decode",
    "test_prefill_fp8_single_query_is_the_decode",
    "test_prefill_int8_chunk_matches_masked_sdpa_on_dequantized_cache",
    "test_prefill_fp8_chunk_matches_masked_sdpa_on_decoded_cache",
    "test_compress_keeps_the_newest_tokens_when_importance_rises",
    "test_compress_keeps_the_prefix_when_importance_falls",
    "test_compress_ties_keep_earlier_tokens_and_nan_ranks_first",
    "test_compress_matches_brute_force_on_tiny_sequences",
    "test_compress_moves_int8_scales_with_their_rows",
    "test_decode_after_compression_equals_attention_over_the_kept_tokens",
    "test_compress_rejects_shared_blocks",
]

RUNNER = r"""
import sys
sys.path.insert(0, {root!r})
import oracle
oracle._default = oracle.OracleLib({path!r})
from tests import test_oracle_pins as PINS
for name in {pins!r}:
    try:
        getattr(PINS, name)()
    except (AssertionError, ValueError, FloatingPointError):
        print("CAUGHT_BY", name)
        sys.exit(1)
print("SURVIVED")
sys.exit(0)
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    assert SRC.count(old) >= 1, f"mutation site for {name} not found"
    path = os.path.join(str(tmp_path), f"liboracle_{name}.so")
    oracle.build_to(path, SRC.replace(old, new))
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    script = RUNNER.format(root=root, path=path, pins=PIN_FUNCS)
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True,
                       timeout=300, env=env)
    # A pin failing (exit 1) or the mutant crashing (killed by a signal) both
    # mean the slip is detected; exit 0 means it survived every pin.
    caught = (r.returncode == 1 and "CAUGHT_BY" in r.stdout) or r.returncode < 0
    assert caught, f"mutant {name} not caught (rc {r.returncode}): {r.stdout[-300:]} {r.stderr[-800:]}"
