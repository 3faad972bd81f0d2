"""The pins catch plausible mistakes: each case below compiles a copy of
oracle.c with one deliberate mistake (a dropped term, a wrong sign, index or
comparison) and checks that at least the named pin fails on it.  The mistakes
live only in temporary copies built on the CPU."""
import os
import shutil
import subprocess

import pytest

import oracle
import test_oracle_attn as A
import test_oracle_commit as C
import test_oracle_commit_inplace as CI
import test_oracle_expand as E
import test_oracle_merge as MG
import test_oracle_probs as PR
import test_oracle_greedy as G
import test_oracle_mss as M
import test_oracle_philox as PH
import test_oracle_topology as T
import test_oracle_varlen as VL

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = [
    # (id, original text, mistaken text, pin that must fail)
    ("topology_self_bit", "for (int j = i; j != -1; j = par[j]) {\n        an[",
     "for (int j = par[i]; j != -1; j = par[j]) {\n        an[",
     lambda: T.test_matches_inverse_of_parent_matrix(8, 2)),
    ("attn_dropped_scale", "s[t] = scale * dot;", "s[t] = dot;",
     lambda: A.test_brute_force_sdpa({})),
    ("attn_head_mapping", "const int h = hq / G;", "const int h = hq % Hkv;",
     A.test_gqa_head_mapping),
    ("attn_lse_missing_max", "lse[r] = m + log(den);", "lse[r] = log(den);",
     A.test_single_key_returns_value_exactly),
    ("attn_path_without_self", "for (int j = i; j != -1; j = par[j]) path[depth++] = j;",
     "for (int j = par[i]; j != -1; j = par[j]) path[depth++] = j;",
     lambda: A.test_brute_force_sdpa({})),
    ("attn_prefix_row_shift", "* Lcap + t) * D;", "* Lcap + t + 1) * D;",
     A.test_chain_is_causal_attention),
    ("greedy_ties_to_highest", "if (row[v] > row[best]) best = v;",
     "if (row[v] >= row[best]) best = v;", G.test_ties_go_to_lowest_index),
    ("greedy_parent_not_required", "acc[c] = acc[par[c]] && tok[c] == amax[par[c]];",
     "acc[c] = tok[c] == amax[par[c]];",
     lambda: [G.test_random_small_trees(s) for s in range(6)]),
    ("greedy_deepest_tie_to_highest", "if (acc[c] && dep[c] > dep[end]) end = c;",
     "if (acc[c] && dep[c] >= dep[end]) end = c;",
     G.test_deepest_accepted_node_wins_over_lower_index),
    ("mss_residual_sign", "float d = fmaf(-s, qc[v], w[v]);",
     "float d = fmaf(s, qc[v], w[v]);",
     lambda: M.test_sample_after_rejection_is_normalised_residual(0)),
    ("mss_mass_dropped_from_test", "const float lhs = (r * qc[x]) * s;",
     "const float lhs = r * qc[x];", M.test_second_child_tested_against_residual),
    ("mss_mass_not_updated", "s = mass(w, V);", "s = 1.0f;",
     M.test_second_child_tested_against_residual),
    ("mss_no_fallback_on_empty_residual",
     "memcpy(w, p_u, sizeof(float) * (size_t)V);\n        break;", "break;",
     M.test_half_q_empties_residual_and_falls_back_to_p),
    ("mss_cdf_not_strict", "if (c > T) return v;", "if (c >= T) return v;",
     M.test_inverse_cdf_end_points),
    ("mss_accept_not_strict", "if (lhs < w[x]) { next = c; break; }",
     "if (lhs <= w[x]) { next = c; break; }", M.test_inverse_cdf_end_points),
    ("philox_one_key_word_bumped", "if (round > 0) { k0 += W0; k1 += W1; }",
     "if (round > 0) { k0 += W0; }", PH.test_matches_numpy_philox),
    ("philox_words_swapped", "n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;",
     "n0 = hi1 ^ c3 ^ k0, n1 = lo1, n2 = hi0 ^ c1 ^ k1, n3 = lo0;", PH.test_matches_numpy_philox),
    ("philox_nine_rounds", "for (int round = 0; round < 10; ++round) {",
     "for (int round = 0; round < 9; ++round) {", PH.test_matches_numpy_philox),
    ("mss_counter_words_swapped", "const uint64_t ctr[4] = {j, (uint64_t)u, (uint64_t)b, step};",
     "const uint64_t ctr[4] = {(uint64_t)u, j, (uint64_t)b, step};",
     lambda: PH.test_seeded_walk_uses_documented_counters(1005, 0, {})),
    ("mss_attempt_ordinal_not_advanced", "      ++j;\n      const float lhs", "\n      const float lhs",
     lambda: PH.test_seeded_walk_uses_documented_counters(3, 2, dict(
         B=64, N=9, tree="star", V=8, prob_sigma=3.0))),
    ("mss_bonus_counter", "#define ORC_BONUS_ORDINAL 0x8000000000000000ull",
     "#define ORC_BONUS_ORDINAL 0x4000000000000000ull",
     lambda: PH.test_seeded_walk_uses_documented_counters(1005, 0, {})),
    ("varlen_attn_validity_over_padding", "if (!tree_is_valid(n, par)) { status[r] = ORC_E_TREE; continue; }",
     "if (!tree_is_valid(N, par)) { status[r] = ORC_E_TREE; continue; }",
     lambda: VL.test_attention_per_request(0)),
    ("varlen_attn_padding_rows_flagged", "if (i >= n) { status[r] = ORC_OK; continue; }",
     "if (i >= n) { status[r] = ORC_E_SHAPE; continue; }",
     lambda: VL.test_attention_per_request(0)),
    ("varlen_topology_padding_walked", "for (int i = 0; i < n; ++i) {\n      int d = -1;",
     "for (int i = 0; i < N && tree_is_valid(N, par); ++i) {\n      int d = -1;",
     lambda: [VL.test_topology_per_request(s) for s in range(4)]),
    ("varlen_greedy_ignores_node_count",
     "int32_t* ob = out_tokens + (size_t)b * N;\n    const int n = nodes_of(n_nodes, b, N);",
     "int32_t* ob = out_tokens + (size_t)b * N;\n    const int n = N;",
     lambda: [VL.test_greedy_per_request(s) for s in range(6)]),
    ("varlen_mss_padding_children", "for (int c = u + 1; c < n; ++c) {",
     "for (int c = u + 1; c < N; ++c) {",
     lambda: [VL.test_stochastic_per_request(s) for s in range(6)]),
    ("expand_ties_to_highest", "(best < 0 || row[v] > row[best])", "(best < 0 || row[v] >= row[best])",
     lambda: [E.test_topk_matches_stable_argsort_with_ties(s) for s in range(5)]),
    ("expand_token_reused", "taken[best] = 1;", "taken[best] = 0;",
     E.test_invariants_and_skipped_frontier_entries),
    ("expand_rank_counts_holes", "if (fb[f] < 0) continue;", "if (fb[f] < 0) { pos += k; continue; }",
     E.test_invariants_and_skipped_frontier_entries),
    ("merge_leader_ignores_length",
     "if (ln[t] >= d && same_prefix(sq + (size_t)t * Ls, sq + (size_t)s * Ls, d)) {",
     "if (same_prefix(sq + (size_t)t * Ls, sq + (size_t)s * Ls, d)) {",
     lambda: [MG.test_brute_force_prefix_sets(s) for s in range(8)]),
    ("merge_prefix_short_by_one", "for (int t = 0; t < d; ++t)\n    if (a[t] != c[t]) return 0;",
     "for (int t = 0; t + 1 < d; ++t)\n    if (a[t] != c[t]) return 0;",
     lambda: [MG.test_brute_force_prefix_sets(s) for s in range(8)]),
    ("merge_parent_same_depth", "pb[next] = node_of[(size_t)s * (Ls + 1) + d - 1];",
     "pb[next] = node_of[(size_t)s * (Ls + 1) + (d > 1 ? d - 2 : 0)];", MG.test_hand_example),
    ("probs_temperature_dropped", "const float c = (float)(ORC_LOG2E / (double)T);",
     "const float c = (float)ORC_LOG2E;", lambda: PR.test_matches_scipy_softmax(0.8)),
    ("probs_ties_to_highest_id", "return i < j ? -1 : (i > j ? 1 : 0);",
     "return i > j ? -1 : (i < j ? 1 : 0);",
     lambda: PR.test_topk_keeps_the_stable_argsort_prefix(5)),
    ("probs_taylor_degree_6", "float p = cf[7];\n  for (int k = 6; k >= 0; --k)",
     "float p = cf[6];\n  for (int k = 5; k >= 0; --k)", PR.test_exp2_against_numpy),
    ("probs_range_reduction_floor", "const float n = rintf(t);", "const float n = floorf(t);",
     PR.test_exp2_against_numpy),
    ("probs_topp_crossing_token_dropped", "        run += mass40(e[order[j]]);\n        ++j;\n        if (run >= need) break;",
     "        if (run + mass40(e[order[j]]) >= need) break;\n        run += mass40(e[order[j]]);\n        ++j;",
     lambda: PR.test_topp_keeps_the_shortest_prefix_reaching_p(0.8, 0, 0.9)),
    ("probs_topp_before_topk", "int kept = (topk > 0 && topk < V) ? topk : V;",
     "int kept = V;",
     lambda: PR.test_topp_keeps_the_shortest_prefix_reaching_p(0.8, 50, 0.95)),
    ("commit_inplace_source_without_length",
     "memcpy(tk + (size_t)j * row, (const char*)k_cache + (base + L + pb[j]) * row, row);",
     "memcpy(tk + (size_t)j * row, (const char*)k_cache + (base + pb[j]) * row, row);",
     lambda: [CI.test_equals_separate_tree_commit(s) for s in range(6)]),
    ("commit_off_by_one", "* Lcap + (L + j)) * row;", "* Lcap + (L + j + 1)) * row;",
     C.test_full_chain_acceptance_appends_tree),
    ("commit_length", "cache_len_out[b] = L + n;", "cache_len_out[b] = L + n - 1;",
     C.test_full_chain_acceptance_appends_tree),
    ("commit_reversed_path", "* N + pb[j]) * row;", "* N + pb[n - 1 - j]) * row;",
     C.test_partial_path_and_canaries),
]


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


@pytest.mark.parametrize("mid,orig,bad,pin", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pin_catches_mutant(mid, orig, bad, pin, mutant_dir):
    src = open(SRC).read()
    assert src.count(orig) == 1, "mutation site must be unique: %r" % orig
    path = os.path.join(str(mutant_dir), mid + ".c")
    open(path, "w").write(src.replace(orig, bad))
    so = os.path.join(str(mutant_dir), "lib" + mid + ".so")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp",
                           "-fPIC", "-shared", "-o", so, path, "-lm"])
    with oracle.use_library(so):
        with pytest.raises(AssertionError):
            pin()


def test_unmutated_copy_passes_the_same_pins(mutant_dir):
    so = os.path.join(str(mutant_dir), "libclean.so")
    shutil.copy(SRC, os.path.join(str(mutant_dir), "clean.c"))
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp",
                           "-fPIC", "-shared", "-o", so,
                           os.path.join(str(mutant_dir), "clean.c"), "-lm"])
    with oracle.use_library(so):
        for _, _, _, pin in MUTANTS:
            pin()
