"""The oracle's pins have teeth: plant a plausible mistake in a copy of the
oracle source (a flipped decision, a transposed ratio, a wrong residual sign
or row, a dropped temperature, a wrong tie rule, a wrong tree recursion...),
build it, and check that at least one pin fails.  Runs on the CPU only; the
mistakes are planted in the oracle, never in GPU code.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "sv_oracle.cpp")

CHAIN_PINS = [
    lambda: pins.test_chain_round_is_lossless(2, 2, 0.6, 0.3, 0.3, 13),
    lambda: pins.test_chain_round_is_lossless(3, 1, 1.0, 0.5, 0.0, 15),
    pins.test_single_step_acceptance_law,
    pins.test_softmax_with_temperature_matches_library,
    pins.test_chain_shaped_tree_is_chain,
    pins.test_greedy_equals_chain_on_one_hot_rows,
]
TREE_PINS = [
    lambda: pins.test_tree_round_with_iid_siblings_is_lossless([-1, 0, 0, 0], 1, 23, 0.8),
    lambda: pins.test_tree_round_with_iid_siblings_is_lossless([-1, 0, 1, 1, 0], 1, 24, 1.3),
    pins.test_chain_shaped_tree_is_chain,
]

PM_CHAIN_PINS = [
    pins.test_pm_chain_equals_chain_with_point_mass_drafts,
    lambda: pins.test_pm_chain_round_is_lossless_for_any_drafter(2, 3, 1.0, 0.0, 41, "p_argmin"),
]
PM_TREE_PINS = [
    lambda: pins.test_pm_tree_with_top_f_siblings_is_lossless([-1, 0, 0, 1, 1], 2, 52, 0.8),
    pins.test_pm_repeated_sibling_token_is_rejected_and_removes_nothing,
    pins.test_pm_chain_shaped_tree_is_pm_chain,
]
CACHE_PINS = [
    pins.test_cache_rank_is_position_in_numpy_stable_order,
    pins.test_cache_rank_brute_force_count,
    pins.test_cache_hit_is_membership_in_the_fanout_cache,
]

PRESTO_PINS = [
    pins.test_presto_scores_match_log_softmax_and_ancestor_sums,
    lambda: pins.test_presto_proxy_minimises_the_kl_objective(1.0),
    pins.test_presto_lambda_zero_expands_the_draft_top_k,
    pins.test_presto_expansion_brute_force,
]

BRANCH_PINS = [pins.test_branch_fork_brute_force, pins.test_branch_fork_special_cases]


MUTANTS = [
    # (name, original text, planted text, pins expected to catch it)
    ("decision inverted", "if (!(r[j] < a)) break;", "if (!(r[j] > a)) break;", CHAIN_PINS),
    ("ratio transposed", "if (qx > 0.0) return px / qx;", "if (px > 0.0) return qx / px;", CHAIN_PINS),
    ("residual sign", "w[v] = std::max(0.0, P[n][v] - Q[n][v]);", "w[v] = std::max(0.0, Q[n][v] - P[n][v]);",
     CHAIN_PINS),
    ("residual row", "w[v] = std::max(0.0, P[n][v] - Q[n][v]);",
     "w[v] = std::max(0.0, P[n + 1][v] - Q[n][v]);", CHAIN_PINS),
    ("bonus row", "    w = P[gamma];\n", "    w = P[gamma - 1];\n", CHAIN_PINS),
    ("temperature dropped", "p[v] = std::exp((load_logit(base, dtype, row_off + v) - M) / T);",
     "p[v] = std::exp(load_logit(base, dtype, row_off + v) - M);", CHAIN_PINS),
    ("softmax not normalised", "  for (int v = 0; v < V; ++v) p[v] /= S;\n", "\n", CHAIN_PINS),
    ("inverse CDF off by one", "      return (int)v;\n    }\n  }\n  int last",
     "      return (int)std::min(v + 1, w.size() - 1);\n    }\n  }\n  int last", CHAIN_PINS),
    ("acceptance counter index", "draw_uniform(seed, (uint32_t)(j + 1), (uint32_t)b, 0, round, 0);",
     "draw_uniform(seed, (uint32_t)j, (uint32_t)b, 0, round, 0);", [pins.test_chain_shaped_tree_is_chain]),
    ("tree recursion step", "const double c_next = c + D;", "const double c_next = c + 1.0;", TREE_PINS),
    ("tree mass not updated", "        D = G;\n", "\n", TREE_PINS),
    ("tree residual not renormalised", "const double pcur = std::max(0.0, p[tok] - c * q[tok]) / D;",
     "const double pcur = std::max(0.0, p[tok] - c * q[tok]);", TREE_PINS),
    ("tree draws from p after rejections", "for (int v = 0; v < in.V; ++v) w[v] = std::max(0.0, p[v] - c * q[v]);",
     "for (int v = 0; v < in.V; ++v) w[v] = p[v];", TREE_PINS),
    ("multi ties to highest k", "if (results[k].n > best_n) {", "if (results[k].n >= best_n) {",
     [pins.test_multi_k1_is_chain_and_each_candidate_is_its_chain]),
    ("multi draws from the first candidate's rows", "out_tok[b] = results[best_k].t;", "out_tok[b] = results[0].t;",
     [pins.test_multi_k1_is_chain_and_each_candidate_is_its_chain]),
    ("multi draws from the last candidate's rows", "out_tok[b] = results[best_k].t;",
     "out_tok[b] = results[K - 1].t;", [pins.test_multi_k1_is_chain_and_each_candidate_is_its_chain]),
    ("greedy ties to highest index", "    if (z > best) {\n      best = z;", "    if (z >= best) {\n      best = z;",
     [pins.test_greedy_ties_lowest_index_and_signed_zero, pins.test_greedy_equals_chain_on_one_hot_rows]),
    ("fan-out unstable order", "std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return z[a] > z[b]; });",
     "std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return z[a] >= z[b] && a != b && z[a] == z[b] ? a > b : z[a] > z[b]; });",
     [pins.test_fanout_is_stable_sort]),
    ("point-mass residual keeps the rejected token", "    w[x[n]] = 0.0;  // the rejected token leaves the residual\n",
     "\n", PM_CHAIN_PINS),
    ("point-mass tree mass not reduced", "      D -= w[tok];\n", "\n", PM_TREE_PINS),
    ("point-mass tree ratio not renormalised", "accept_ratio(w[tok] / D, 1.0)", "accept_ratio(w[tok], 1.0)",
     PM_TREE_PINS),
    ("point-mass tree draw ignores removals", "    if (!(mass > 0.0)) w = p;\n", "    w = p;\n", PM_TREE_PINS),
    ("cache rank ties to the highest index", "(z[a] == z[c] && a < c)", "(z[a] == z[c] && a > c)", CACHE_PINS),
    ("cache hit counts the F-th token in", "out_hit[b] = pos < F[n[b]] ? 1 : 0;",
     "out_hit[b] = pos <= F[n[b]] ? 1 : 0;", CACHE_PINS),
    ("cache row of the next position", "const int64_t row = (int64_t)b * (K + 1) + n[b];",
     "const int64_t row = (int64_t)b * (K + 1) + (n[b] < K ? n[b] + 1 : n[b]);", CACHE_PINS),
    ("presto ratio not clipped at 1", "const double rho = std::min(1.0, p / q);", "const double rho = p / q;",
     PRESTO_PINS),
    ("presto lambda on the draft term", "return logq + lambda * std::log(rho);",
     "return lambda * logq + std::log(rho);", PRESTO_PINS),
    ("presto path score drops the parent", "S_b[i] = S_b[par[i]] + s_b[i];", "S_b[i] = s_b[i];", PRESTO_PINS),
    ("presto expands internal nodes too", "      if (nkids[u] == 0) {\n", "      if (nkids[u] >= 0) {\n",
     PRESTO_PINS),
    ("presto expansion uses the leaf's own depth", "presto_lambda(lam, D, depth[u] + 1)",
     "presto_lambda(lam, D, depth[u] > 0 ? depth[u] : 1)", PRESTO_PINS),
    ("branch point at the first confident token", "        if (qx < eps) {", "        if (qx > eps) {",
     BRANCH_PINS),
    ("branch count rounded up", "std::max(1, (int)std::floor(kf));", "std::max(1, (int)std::ceil(kf));", BRANCH_PINS),
    ("branch count ignores confidence", "const double kf = (double)k_max * (1.0 - qb);",
     "const double kf = (double)k_max * qb;", BRANCH_PINS),
    ("class 0 branches at the next round", "    if (s == 0) {\n      pos = 1;", "    if (s == 0) {\n      pos = gamma + 1;",
     BRANCH_PINS),
    ("geometric fan-out floor", "F_out[k] = (int32_t)std::ceil(f);", "F_out[k] = (int32_t)std::floor(f);",
     [pins.test_geometric_fanout_closed_form]),
]


@pytest.mark.parametrize("name,old,new,catchers", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, catchers):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for '{name}' not unique"
    mutant = tmp_path / "mutant.cpp"
    mutant.write_text(src.replace(old, new))
    so = str(tmp_path / "libmutant.so")
    subprocess.run(["g++", "-O1", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off", str(mutant), "-o", so],
                   check=True)
    caught = []
    with oracle.use_library(so):
        for pin in catchers:
            try:
                pin()
            except (AssertionError, oracle.OracleError):
                caught.append(pin)
    assert caught, f"no pin caught the planted mistake '{name}'"
