"""The pins have teeth: a plausible mistake planted in a copy of the oracle
source makes at least one of the named pins fail.

Every mistake is planted in the oracle, on the CPU (a temporary copy of the C
source, compiled with gcc); nothing here touches the HIP path.
"""
import os

import pytest

import oracle
import pins

# (name, source snippet, replacement, pins expected to catch it)
MUTANTS = [
    ("naive_resample_from_p", "r[v] = diff > 0.0 ? diff : 0.0;", "r[v] = pm[v];",
     ["three_option_grid", "chisq_v8_g4"]),
    ("non_strict_accept", "if (!(ua[i] < acc_p)) break;", "if (!(ua[i] <= acc_p)) break;",
     ["strict_comparisons"]),
    ("greedy_rows_shifted",
     "g = row_argmax(row_ptr(target, a->is_bf16, (int64_t)b * (G + 1) + i, V), a->is_bf16, V);",
     "g = row_argmax(row_ptr(target, a->is_bf16, (int64_t)b * (G + 1) + (i < gb ? i + 1 : i), V),"
     " a->is_bf16, V);",
     ["greedy_walkthrough", "greedy_matches_numpy"]),
    ("sampling_rows_shifted",
     "oracle_row_distribution(row_ptr(target, a->is_bf16, (int64_t)b * (G + 1) + i, V),",
     "oracle_row_distribution(row_ptr(target, a->is_bf16, (int64_t)b * (G + 1)"
     " + (i < gb ? i + 1 : i), V),",
     ["chisq_v8_g4", "chisq_v16_g4"]),
    ("temperature_dropped", "/ T", "/ 1.0", ["probabilities_logsumexp"]),
    ("philox_multiplier", "0xD2511F53u", "0xD2511F55u", ["philox_kat"]),
    ("philox_key_bump", "k1 += 0xBB67AE85u;", "k1 += 0xBB67AE86u;", ["philox_kat"]),
    ("greedy_tie_highest_index", "if (z > best_z)", "if (z >= best_z)",
     ["greedy_walkthrough", "greedy_matches_numpy"]),
    ("residual_next_draft_row", "const double* qm = Q + (size_t)m * V;",
     "const double* qm = Q + (size_t)(m + 1 < gb ? m + 1 : m) * V;",
     ["chisq_v8_g4", "chisq_v16_g4"]),
    ("bonus_from_draft",
     "for (int64_t v = 0; v < V; ++v) { r[v] = pm[v]; R += r[v]; }\n"
     "                if (residual_mass) residual_mass[k] = 0.0;",
     "for (int64_t v = 0; v < V; ++v) { r[v] = Q[(size_t)(gb > 0 ? gb - 1 : 0) * V + v];"
     " R += r[v]; }\n                if (residual_mass) residual_mass[k] = 0.0;",
     ["expected_advance"]),
    ("cdf_non_strict", "if (C > target_mass)", "if (C >= target_mass)",
     ["strict_comparisons"]),
    ("near_accept_not_noted", "if (fabs(ua[i] - acc_p) < NEAR_EPS) note_near(&near, i);",
     "if (0) note_near(&near, i);", ["near_threshold"]),
    ("near_draw_not_noted",
     "if (fabs(us[m] - C_prev / R) < NEAR_EPS || fabs(us[m] - C / R) < NEAR_EPS)",
     "if (0)", ["near_threshold"]),
    ("near_window_too_wide", "#define NEAR_EPS 1e-6", "#define NEAR_EPS 1e-5", ["near_threshold"]),
    ("same_uniform_for_sampling", "*u_sample = (double)(w[1] >> 8)", "*u_sample = (double)(w[0] >> 8)",
     ["chisq_v8_g4", "chisq_v16_g4", "chisq_v3_g1"]),
    ("topk_drops_ties", "keep[v] = logit_at(row, is_bf16, v) >= tau;",
     "keep[v] = logit_at(row, is_bf16, v) > tau;", ["truncation"]),
    ("topp_cut_one_short", "if (cum >= top_p) { cut = j; break; }",
     "if (cum >= top_p) { cut = j > 0 ? j - 1 : 0; break; }", ["truncation"]),
    ("topp_not_renormalized", "if (keep[v]) S2 += exp(", "if (1) S2 += exp(", ["truncation"]),
    ("commit_drops_last_accepted", "if (j <= m) {", "if (j < m) {", ["commit_numpy"]),
    ("commit_length_t_plus_m", "seq_lens[b] = seq_lens[b] + accept_count[b] + 1;",
     "seq_lens[b] = seq_lens[b] + accept_count[b];", ["commit_numpy"]),
    ("residual_sign_flipped", "double diff = pm[v] - qm[v];", "double diff = qm[v] - pm[v];",
     ["three_option_grid", "invariants"]),
    ("eos_itself_dropped", "if (e >= 0) n = e + 1;", "if (e >= 0) n = e;",
     ["round_end_walkthrough", "round_end_autoregressive"]),
    ("eos_search_skips_drawn_token", "for (int32_t j = 0; j <= m; ++j)\n            if (out[j] == eos)",
     "for (int32_t j = 0; j < m; ++j)\n            if (out[j] == eos)",
     ["round_end_walkthrough", "round_end_autoregressive"]),
    ("budget_one_too_many", "n = budget;", "n = budget + 1 < m + 1 ? budget + 1 : m + 1;",
     ["round_end_walkthrough", "round_end_prefix"]),
    ("accept_count_not_cut", "*kept_m = m < n ? m : n;", "*kept_m = m;",
     ["round_end_walkthrough", "round_end_autoregressive"]),
    ("rollback_keeps_first_rejected", "for (int32_t j = m + 1; j < gb; ++j) {",
     "for (int32_t j = m + 2; j < gb; ++j) {", ["rollback_invariants"]),
    ("rollback_length_past_written",
     "const int32_t keep = accept_count[b] + 1 < gb ? accept_count[b] + 1 : gb;",
     "const int32_t keep = accept_count[b] + 1;", ["rollback_invariants"]),
    ("tree_node_judged_by_its_own_row", "ok[j] = ok[par[j]] && tok[j] == choice[par[j]];",
     "ok[j] = ok[par[j]] && tok[j] == choice[j];", ["tree_walkthrough", "tree_brute_force"]),
    ("tree_ignores_parent_rejection", "ok[j] = ok[par[j]] && tok[j] == choice[par[j]];",
     "ok[j] = tok[j] == choice[par[j]];", ["tree_walkthrough", "tree_brute_force"]),
    ("tree_tie_to_highest_node", "if (ok[j] && depth[j] > depth[best]) best = j;",
     "if (ok[j] && depth[j] >= depth[best]) best = j;", ["tree_walkthrough", "tree_brute_force"]),
    ("tree_next_token_from_parent_row", "out[m] = choice[best];",
     "out[m] = choice[best ? par[best] : 0];", ["tree_walkthrough", "tree_chain_equals_chain"]),
    ("commit_ignores_slot_map",
     "const int32_t slot = slot_map ? slot_map[(size_t)b * (G + 1) + j] : j;",
     "const int32_t slot = j;", ["commit_slot_map"]),
    ("ngram_earliest_occurrence",
     "for (int32_t s = L - n - 1; s >= 0 && found < 0; --s) {",
     "for (int32_t s = 0; s <= L - n - 1 && found < 0; ++s) {",
     ["ngram_worked_cases", "ngram_brute_force"]),
    ("ngram_shortest_first", "for (int32_t n = n_max; n >= n_min; --n) {",
     "for (int32_t n = n_min; n <= n_max; ++n) {", ["ngram_worked_cases", "ngram_brute_force"]),
    ("ngram_matches_itself", "for (int32_t s = L - n - 1; s >= 0 && found < 0; --s) {",
     "for (int32_t s = L - n; s >= 0 && found < 0; --s) {",
     ["ngram_worked_cases", "ngram_brute_force"]),
    ("ngram_skips_next_token", "const int32_t first = found + n;",
     "const int32_t first = found + n + 1;", ["ngram_worked_cases", "ngram_brute_force"]),
    ("point_mass_misplaced", "if (d[i] >= 0 && d[i] < V) Q[(size_t)i * V + d[i]] = 1.0;",
     "if (d[i] >= 0 && d[i] < V) Q[(size_t)i * V + (d[i] + 1) % V] = 1.0;",
     ["point_mass_acceptance"]),
    ("point_mass_untruncated_target",
     "a->is_bf16, V, a->temperature, a->top_k, a->top_p,\n"
     "                                        P + (size_t)i * V, &nc);",
     "a->is_bf16, V, a->temperature, draft ? a->top_k : 0, draft ? a->top_p : 1.0,\n"
     "                                        P + (size_t)i * V, &nc);",
     ["point_mass_truncated"]),
]


@pytest.mark.parametrize("name,old,new,catchers", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new, catchers, tmp_path):
    src = open(oracle.SRC).read()
    count = src.count(old)
    assert count >= 1, f"snippet for {name} not found in the oracle source"
    if name != "temperature_dropped":
        assert count == 1, f"snippet for {name} is ambiguous ({count} matches)"
    mutant = oracle.build_copy(src.replace(old, new), str(tmp_path / name))
    caught = {c: pins.ALL_PINS[c](mutant) for c in catchers}
    assert any(caught.values()), f"no pin caught the planted mistake {name}: {caught}"
