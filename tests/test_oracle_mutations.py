"""The oracle's pins have teeth: each test plants one plausible mistake in a
copy of the oracle's C source, builds it, swaps it in, and checks that a pin
fails. Mistakes are planted on the CPU only, in a temporary copy; the real
oracle is restored after each case."""
import contextlib
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
import test_bandit_oracle as bandit
import test_oracle_lowrank as lowrank
import test_oracle_tree as tree
import test_oracle_tree_sample as tsample
import test_oracle_outcomes as outcomes
import test_oracle_pins as pins
import test_oracle_stats as stats

ORACLE_DIR = os.path.dirname(oracle.__file__)
SRC = os.path.join(ORACLE_DIR, "spec_oracle.c")
BANDIT_SRC = os.path.join(ORACLE_DIR, "bandit_oracle.c")


@contextlib.contextmanager
def mutated_oracle(old: str, new: str, target: str = SRC):
    """Build the oracle library with one mistake planted in ``target``."""
    text = open(target).read()
    assert text.count(old) >= 1, f"mutation anchor not found: {old!r}"
    d = tempfile.mkdtemp(prefix="oracle_mut_")
    srcs = []
    for path in (SRC, BANDIT_SRC):
        out = os.path.join(d, os.path.basename(path))
        body = open(path).read()
        with open(out, "w") as f:
            f.write(body.replace(old, new) if path == target else body)
        srcs.append(out)
    lib = os.path.join(d, "libm_oracle.so")
    subprocess.run(["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-o", lib,
                    *srcs, "-lm"], check=True, capture_output=True)
    saved_lib, saved_path = oracle._lib, oracle.LIB_PATH
    oracle._lib = None
    oracle.LIB_PATH = lib
    try:
        oracle._load()
        yield
    finally:
        oracle._lib, oracle.LIB_PATH = saved_lib, saved_path
        shutil.rmtree(d, ignore_errors=True)


def fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_residual_without_the_max_is_caught():
    with mutated_oracle("r[v] = p - q > 0.0 ? p - q : 0.0;", "r[v] = p;"):
        fails(pins.test_residual_distribution_exact_sweep, 1.0)


def test_flipped_accept_ratio_is_caught():
    with mutated_oracle("int accept = log_u < (lp - lq);", "int accept = log_u < (lq - lp);"):
        fails(pins.test_accept_probability_exact_sweep, 1.0)


def test_temperature_ignored_is_caught():
    with mutated_oracle("float x = z * inv_t;", "float x = z;"):
        fails(pins.test_row_lse_matches_scipy, "f32", 0.7)


def test_philox_constant_typo_is_caught(torch_philox_exe):
    with mutated_oracle("const uint32_t M0 = 0xD2511F53u", "const uint32_t M0 = 0xD2511F55u"):
        fails(pins.test_philox_matches_library_engine, torch_philox_exe)


def test_philox_round_count_is_caught(torch_philox_exe):
    with mutated_oracle("round < 10; ++round", "round < 7; ++round"):
        fails(pins.test_philox_matches_library_engine, torch_philox_exe)


def test_inclusive_bin_edge_is_caught():
    with mutated_oracle("if (prefix > tau) {", "if (prefix >= tau) {"):
        fails(pins.test_inverse_cdf_worked_margins)


def test_lse_without_max_shift_is_caught():
    with mutated_oracle("s += exp(x - m);\n    }\n    return m + log(s);",
                        "s += exp(x - m + 1e-3);\n    }\n    return m + log(s);"):
        fails(pins.test_row_lse_closed_forms)


def test_last_index_on_ties_is_caught():
    with mutated_oracle("if (z > best_z) {", "if (z >= best_z) {"):
        fails(pins.test_row_argmax_first_index_on_ties)


def test_bonus_from_the_wrong_row_is_caught():
    # the bonus (all accepted) draws from target row G; use row G-1 instead
    with mutated_oracle("p_row0 + (size_t)k * V, k == G, inv_t, k < G ? lse_q[k] : 0.0,\n                          lse_p[k],",
                        "p_row0 + (size_t)(k == G && k > 0 ? k - 1 : k) * V, k == G, inv_t,\n                          k < G ? lse_q[k] : 0.0, lse_p[k == G && k > 0 ? k - 1 : k],"):
        fails(pins.test_bonus_distribution_exact_sweep)


def test_marginal_gate_catches_a_biased_residual():
    """The statistical gate alone (chi-square over 10,000 draws) also catches
    drawing the correction from p instead of the residual."""
    with mutated_oracle("r[v] = p - q > 0.0 ? p - q : 0.0;", "r[v] = p;"):
        fails(stats.test_gate_output_marginal_is_target, stats.build_gate_case())


def test_outcome_length_law_without_the_reject_factor_is_caught():
    with mutated_oracle("pk_b[i] = i < G ? reach * (1.0 - beta[i]) : reach;",
                        "pk_b[i] = reach;"):
        fails(outcomes.test_outcome_law_matches_the_verification_oracle, (0.6, 0.6, 0.6))


def test_outcome_acceptance_without_the_cap_is_caught():
    with mutated_oracle("beta[j] = d >= 0.0 ? 1.0 : (d < 0.0 ? exp(d) : 0.0);",
                        "beta[j] = d == d ? exp(d) : 0.0;"):
        fails(outcomes.test_outcome_law_matches_the_verification_oracle, (0.6, 1.8, 0.4))


def test_outcome_top_f_last_index_on_ties_is_caught():
    with mutated_oracle("if (best < 0 || r[v] > r[best])", "if (best < 0 || r[v] >= r[best])"):
        fails(outcomes.test_top_f_is_the_stable_sort_of_the_distribution)


def test_outcome_residual_without_the_max_is_caught():
    with mutated_oracle("r[v] = p - q > 0.0 ? p - q : 0.0;\n                        sc[v] = p + q;",
                        "r[v] = p - q;\n                        sc[v] = p + q;"):
        fails(outcomes.test_residual_mass_is_total_variation)


def test_head_up_projection_transposed_is_caught():
    with mutated_oracle("double t = (double)bf16_bits_to_float(w_up[(size_t)v * r + j]) * uu[j];",
                        "double t = (double)bf16_bits_to_float(w_up[(size_t)j * V + v]) * uu[j];"):
        fails(lowrank.test_products_match_numpy)


def test_head_activation_not_rounded_is_caught():
    with mutated_oracle("uu[j] = (double)bf16_bits_to_float(u[(size_t)i * r + j]);", "uu[j] = s;"):
        fails(lowrank.test_products_match_numpy)


def test_head_normaliser_without_temperature_is_caught():
    with mutated_oracle("lse[i] = oracle_row_lse(z + (size_t)i * V, ORACLE_BF16, 0, V, inv_t);",
                        "lse[i] = oracle_row_lse(z + (size_t)i * V, ORACLE_BF16, 0, V, 1.0f);"):
        fails(lowrank.test_lse_matches_scipy)


def test_head_ties_to_odd_are_caught():
    with mutated_oracle("(e1 == e0 && (n & 1u) == 0u)", "(e1 == e0 && (n & 1u) == 1u)"):
        fails(lowrank.test_bf16_rounding_matches_torch_and_ties_go_to_even)


def test_tree_score_without_the_path_is_caught():
    with mutated_oracle("c[i] = c[par[i]] + (double)lq[i];", "c[i] = (double)lq[i];"):
        fails(tree.test_path_scores_and_kept_set_by_brute_force)


def test_tree_ties_to_the_higher_index_are_caught():
    with mutated_oracle("if (c[j] > c[i] || (c[j] == c[i] && j < i))",
                        "if (c[j] > c[i] || (c[j] == c[i] && j > i))"):
        fails(tree.test_prune_ties_go_to_the_lower_index)


def test_tree_walk_taking_the_last_match_is_caught():
    with mutated_oracle("""                if (par[j] == x && tk[j] == a) {
                    next = j;
                    break;
                }""", """                if (par[j] == x && tk[j] == a)
                    next = j;"""):
        fails(tree.test_greedy_tree_duplicate_siblings_take_the_lower_index)


def test_tree_extra_token_from_the_root_is_caught():
    with mutated_oracle("                extra[b] = a;\n", "                extra[b] = oracle_row_argmax(target, dtype, ((size_t)b * M) * V, V);\n"):
        fails(tree.test_greedy_tree_on_chains_matches_the_verifier)


def ucb1_pins():
    run = bandit.run_bandits(oracle.UCB1, seeds=24, rounds=10_000, snapshot=1_000)
    bandit.test_ucb1_regret_within_auer_bound(run)
    bandit.test_ucb1_regret_grows_logarithmically(run)


def thompson_pins():
    bandit.test_gamma_sampler_matches_scipy()
    bandit.test_beta_sampler_matches_scipy()
    bandit.test_thompson_choice_probabilities_match_the_posterior()
    run = bandit.run_bandits(oracle.THOMPSON, seeds=24, rounds=10_000, snapshot=1_000)
    bandit.test_thompson_regret_logarithmic_and_below_ucb1_bound(run)


def test_ucb1_bonus_with_the_wrong_sign_is_caught():
    with mutated_oracle("score[j] = mean + bonus;", "score[j] = mean - bonus;", BANDIT_SRC):
        fails(ucb1_pins)


def test_ucb1_sum_in_place_of_mean_is_caught():
    with mutated_oracle("double mean = sums[j] / nj;", "double mean = sums[j];", BANDIT_SRC):
        fails(ucb1_pins)


def test_ucb1_without_log_of_plays_is_caught():
    with mutated_oracle("sqrt(2.0 * log((double)n) / nj)", "sqrt(2.0 / nj)", BANDIT_SRC):
        fails(ucb1_pins)


def test_marsaglia_tsang_without_the_third_is_caught():
    with mutated_oracle("const double d = shape - 1.0 / 3.0;", "const double d = shape;",
                        BANDIT_SRC):
        fails(thompson_pins)


def test_box_muller_reusing_a_uniform_is_caught():
    with mutated_oracle("cos(two_pi * u2)", "cos(two_pi * u1)", BANDIT_SRC):
        fails(thompson_pins)


def test_thompson_failures_counted_as_plays_is_caught():
    with mutated_oracle("double b = 1.0 + ((double)counts[j] - sums[j]);",
                        "double b = 1.0 + (double)counts[j];", BANDIT_SRC):
        fails(thompson_pins)


def test_reward_not_divided_by_gamma_is_caught():
    with mutated_oracle("double r = (double)ksum / ((double)gamma * (double)m);",
                        "double r = (double)ksum / (double)m;", BANDIT_SRC):
        fails(bandit.test_bandit_skips_invalid_rows_and_bad_arms)


@pytest.fixture(scope="module")
def torch_philox_exe():
    d = tempfile.mkdtemp(prefix="philox_mut_")
    yield pins.build_torch_philox_exe(d)
    shutil.rmtree(d, ignore_errors=True)


def test_tree_sampling_without_the_residual_update_is_caught():
    # the next child is tested against p again instead of the residual
    with mutated_oracle("""                    wsum = sum;
                    residual = 1;""", """                    wsum = sum;
                    residual = 0;"""):
        fails(tsample.test_outputs_follow_the_target)


def test_tree_sampling_residual_the_wrong_way_is_caught():
    with mutated_oracle("""                        const double r = cur - q[v];
                        w[v] = r > 0.0 ? r : 0.0;""", """                        const double r = q[v] - cur;
                        w[v] = r > 0.0 ? r : 0.0;"""):
        fails(tsample.test_outputs_follow_the_target)


def test_tree_sampling_uniform_block_off_by_one_is_caught():
    with mutated_oracle("oracle_philox_words(seed, offset, sid, s - 1, words);",
                        "oracle_philox_words(seed, offset, sid, s, words);"):
        fails(tsample.test_chain_is_the_verifier, 2, dict())


def test_neighbour_on_the_wrong_side_is_caught():
    with mutated_oracle("if (lower <= upper) {", "if (lower > upper) {"):
        fails(pins.test_inverse_cdf_alt_is_the_draw_just_across_the_edge)


def test_neighbour_that_keeps_zero_weights_is_caught():
    with mutated_oracle("for (int v = j - 1; v >= 0; --v)\n                        if (r[v] > 0.0) {",
                        "for (int v = j - 1; v >= 0; --v)\n                        if (r[v] >= 0.0) {"):
        fails(pins.test_inverse_cdf_alt_worked_neighbours)


def test_fanout_ties_to_the_higher_length_are_caught():
    with mutated_oracle("if (best < 0 || v > best_v) {", "if (best < 0 || v >= best_v) {"):
        fails(outcomes.fanout_diagonals)


def test_fanout_without_the_length_probability_is_caught():
    with mutated_oracle("double v = (double)pk_b[i] * (double)pr_b[(size_t)i * F + n[i]];",
                        "double v = (double)pr_b[(size_t)i * F + n[i]];"):
        fails(outcomes.fanout_is_optimal)
