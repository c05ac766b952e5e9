"""Plants plausible mistakes in a copy of the oracle's C source and checks that
the pins in test_oracle.py catch every one of them (no GPU).

Each mutant is a one-line textual change of pa_oracle.c compiled into a
temporary library; the pin battery then runs against that library.  A mutant
"survives" if every pin still passes — that would mean the pins cannot tell
the mistake from the correct oracle, and the test fails.
"""
import importlib.util
import os
import subprocess

import pytest
import torch

import oracle as real_oracle
import test_oracle as pins

SRC = os.path.join(os.path.dirname(real_oracle.__file__), "pa_oracle.c")
INIT = os.path.join(os.path.dirname(real_oracle.__file__), "__init__.py")

MUTANTS = {
    "causal_off_by_one": ("          int end = pos + 1;", "          int end = pos;"),
    "full_mask_still_causal": ("          if (mask == ORC_MASK_FULL) end = L;", ""),
    "sink_weights_not_shrunk": ("              for (int d = 0; d < Dv; ++d) o[d] *= wr / (wr + ws);\n", ""),
    "sink_lse_unchanged": ("              l_out = mx + log(wr + ws);\n", ""),
    "sink_without_max_shift": ("const double wr = exp(l_out - mx), ws = exp(sk - mx);",
                               "const double wr = exp(l_out), ws = exp(sk);"),
    "prefix_capped_one_short": ("            end = prefix_lens[b] < L ? prefix_lens[b] : L;",
                                "            end = prefix_lens[b] < L ? prefix_lens[b] : L - 1;"),
    "prefix_off_by_one": ("if (mask == ORC_MASK_PREFIX && prefix_lens[b] > end)\n            end = prefix_lens[b] < L ? prefix_lens[b] : L;",
                          "if (mask == ORC_MASK_PREFIX && prefix_lens[b] > end)\n            end = prefix_lens[b] + 1 < L ? prefix_lens[b] + 1 : L;"),
    "scale_dropped": ("s[t] = sigma * dot + alibi_bias(", "s[t] = dot + alibi_bias("),
    "alibi_sign_flipped": ("if (mode == ORC_ALIBI_LINEAR) return -slope * dist;",
                           "if (mode == ORC_ALIBI_LINEAR) return slope * dist;"),
    "alibi_sqrt_dropped": ("if (mode == ORC_ALIBI_SQRT) return -slope * sqrt(dist);",
                           "if (mode == ORC_ALIBI_SQRT) return -slope * dist;"),
    "alibi_distance_off_by_one": ("fabs((double)pos - (double)t)", "fabs((double)pos - (double)t + 1.0)"),
    "alibi_slope_of_kv_head": ("alibi_mode ? (double)alibi_slopes[hh] : 0.0",
                               "alibi_mode ? (double)alibi_slopes[h] : 0.0"),
    "alibi_token_index_for_position": ("alibi_mode ? (double)alibi_slopes[hh] : 0.0, pos, s,",
                                       "alibi_mode ? (double)alibi_slopes[hh] : 0.0, j, s,"),
    "gqa_head_ignored": ("key_index(layout, page, slot, h, d, Hkv, P, Dqk)",
                         "key_index(layout, page, slot, 0, d, Hkv, P, Dqk)"),
    "value_layout_transposed": ("return (((size_t)page * Hkv + head) * Dv + d) * P + slot;",
                                "return (((size_t)page * Hkv + head) * P + slot) * Dv + d;"),
    "slot_reversed": ("int slot = t % P;", "int slot = (P - 1) - t % P;"),
    "merge_without_max_shift": ("double w = exp(ls[s] - M);", "double w = exp(ls[s]);"),
    "lse_drops_max": ("*lse = m + log(l);", "*lse = log(l);"),
    "split_not_page_aligned": ("int per = P * ((pages + S - 1) / S);", "int per = (L + S - 1) / S;"),
    "value_read_from_key_cache": ("vc, dtype, value_index(", "kc, dtype, value_index("),
    "no_normalisation": ("for (int d = 0; d < Dv; ++d) out[d] /= l;", ""),
    "block_table_row_stride": ("block_table + (size_t)b * max_pages,\n               num_pages, L, h,",
                               "block_table + (size_t)b,\n               num_pages, L, h,"),
    "empty_partition_lse_zero": ("    *lse = -INFINITY;\n    return;", "    *lse = 0.0;\n    return;"),
    "query_head_index": ("qrow[d] = load_elem(q, dtype, ((size_t)i * Hq + hh) * Dqk + d);",
                         "qrow[d] = load_elem(q, dtype, ((size_t)i * Hq + h) * Dqk + d);"),
    "mla_value_tail_columns": ("  if (layout == ORC_LAYOUT_MLA) return ((size_t)page * P + slot) * Dqk + d;\n"
                               "  return (((size_t)page * Hkv + head) * Dv + d) * P + slot;",
                               "  if (layout == ORC_LAYOUT_MLA) return ((size_t)page * P + slot) * Dqk + d + (Dqk - Dv);\n"
                               "  return (((size_t)page * Hkv + head) * Dv + d) * P + slot;"),
    "merge_weight_sum_skipped": ("      wsum += w;\n", "      wsum += 1.0;\n"),
    "chunk_ignores_causal_limit": ("            if (t1 > seen) t1 = seen;", "            if (t1 > L) t1 = L;"),
    "chunk_start_one_chunk_late": ("long t0 = (long)sp * C, t1 = t0 + C;", "long t0 = (long)(sp + 1) * C, t1 = t0 + C;"),
}


def _battery():
    """Every pin of test_oracle.py, as (name, thunk) pairs."""
    out = []
    for case in pins.CASES:
        for dt in (torch.float32, torch.bfloat16):
            out.append(("sdpa", lambda c=case, d=dt: pins.test_bruteforce_against_torch_sdpa(c, d)))
    for S in (1, 2, 3, 7, 64):
        out.append(("split", lambda s=S: pins.test_split_then_merge_equals_unsplit(s)))
    for pf in ([0, 5, 9, 3, 20, 2], [1, 13, 13, 6, 33, 12], [2, 40, 1, 4, 7, 11]):
        out.append(("prefix", lambda p=pf: pins.test_prefix_mask_matches_sdpa(p)))
    for C in (1, 3, 4, 16, 64):
        out.append(("chunked", lambda c=C: pins.test_chunked_then_merge_equals_unchunked(c)))
    for mode in (real_oracle.ALIBI_LINEAR, real_oracle.ALIBI_SQRT):
        for mask, pf in ((real_oracle.MASK_CAUSAL, None), (real_oracle.MASK_FULL, None),
                         (real_oracle.MASK_PREFIX, [2, 13, 13, 6, 33, 12])):
            out.append(("alibi", lambda m=mode, k=mask, p=pf:
                        pins.test_alibi_matches_sdpa_with_an_additive_bias(m, k, p)))
    for name in ("test_page_permutation_is_bitwise_invariant",
                 "test_split_partials_match_sdpa_on_their_ranges",
                 "test_chunked_partials_match_sdpa_on_visible_keys",
                 "test_full_mask_equals_unmasked_sdpa",
                 "test_mask_special_cases_reduce_to_causal_or_full",
                 "test_sinks_match_sdpa_with_an_extra_zero_key",
                 "test_alibi_zero_slopes_change_nothing",
                 "test_alibi_decode_equals_last_prefill_row",
                 "test_minus_infinite_sinks_change_nothing",
                 "test_constant_value_rows_sum_to_one", "test_length_one_context_returns_v0",
                 "test_equal_keys_give_mean_of_visible_values",
                 "test_zero_query_gives_mean_and_log_count",
                 "test_decode_equals_last_prefill_row_and_extend_matches_prefill",
                 "test_gqa_equals_replicated_mha", "test_request_order_permutation",
                 "test_mla_latent_layout_matches_sdpa_and_mha_layout",
                 "test_merge_closed_forms"):
        out.append((name, getattr(pins, name)))
    for ex in pins._load_golden():
        out.append(("golden", lambda e=ex: pins.test_hand_worked_examples(e)))
    return out


def _mutant_module(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor for %s not found" % name
    msrc = tmp_path / ("m_%s.c" % name)
    msrc.write_text(src.replace(old, new))
    so = tmp_path / ("libm_%s.so" % name)
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-w",
                           "-o", str(so), str(msrc), "-lm"])
    spec = importlib.util.spec_from_file_location("oracle_mutant_" + name, INIT)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._LIB = str(so)
    mod._SRC = str(msrc)
    mod._lib = None
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_kill_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    mod = _mutant_module(tmp_path, name, old, new)
    saved = pins.oracle
    pins.oracle = mod
    caught = []
    try:
        for pin, fn in _battery():
            try:
                fn()
            except (AssertionError, ValueError):
                caught.append(pin)
    finally:
        pins.oracle = saved
    assert caught, "mutant %r survived every pin" % name


def test_unmutated_copy_passes_battery(tmp_path):
    """Control: the same harness with no mutation passes every pin."""
    mod = _mutant_module(tmp_path, "none", "int orc_max_threads(void) {",
                         "int orc_max_threads(void) {")
    saved = pins.oracle
    pins.oracle = mod
    try:
        for pin, fn in _battery():
            fn()
    finally:
        pins.oracle = saved
