"""Planted mistakes in the oracle, on the CPU: each mutant of oracle.c must be
caught by the pin suite (tests/test_oracle_pins.py). This shows the pins are
strong enough that a plausible slip (a dropped term, a flipped sign, a wrong
row index, a wrong constant) cannot pass unnoticed."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "residual_sign": ("r[j] = fmax(0.0, pk[j] - qk[j]);", "r[j] = fmax(0.0, qk[j] - pk[j]);"),
    "accept_flip": ("if (u < alpha) {", "if (u > alpha) {"),
    "row_off_by_one": ("double p = P[(size_t)i * V + x];", "double p = P[(size_t)(i + 1) * V + x];"),
    "ratio_inverted": ("else alpha = fmin(1.0, p / q);", "else alpha = fmin(1.0, q / p);"),
    "bonus_from_wrong_row": ("for (int64_t j = 0; j < V; ++j) r[j] = pk[j];",
                             "for (int64_t j = 0; j < V; ++j) r[j] = P[(size_t)(gamma - 1) * V + j];"),
    "temperature_dropped": ("double e = exp(widen(row, dtype, j) / T - M);",
                            "double e = exp(widen(row, dtype, j) - mx);"),
    "greedy_last_tie": ("if (l > best) { best = l; at = j; }", "if (l >= best) { best = l; at = j; }"),
    "philox_weyl": ("PHILOX_WEYL1 = 0xBB67AE85u", "PHILOX_WEYL1 = 0xBB67AE87u"),
    "uniform_words": ("(((uint64_t)x[1] << 32) | (uint64_t)x[0]) >> 11",
                      "(((uint64_t)x[3] << 32) | (uint64_t)x[2]) >> 11"),
    "sample_uses_accept_uniform": ("us[b * (gamma + 1) + k] = orc_uniform(seed, gb, (uint32_t)k, ORC_PURPOSE_SAMPLE);",
                                   "us[b * (gamma + 1) + k] = orc_uniform(seed, gb, (uint32_t)k, ORC_PURPOSE_ACCEPT);"),
    "no_early_stop": ("            k = i;\n            break;\n        }\n    }\n    if (k == gamma && !usable[gamma])",
                      "            if (k == gamma) k = i;\n        }\n    }\n    if (k == gamma && !usable[gamma])"),
    "draft_purpose": ("ORC_PURPOSE_DRAFT)\n", "ORC_PURPOSE_SAMPLE)\n"),
    "draft_position": ("(uint32_t)(b + b_offset), (uint32_t)(pos0 + t),", "(uint32_t)(b + b_offset), (uint32_t)(t),"),
    "draft_sequence": ("(uint32_t)(b + b_offset), (uint32_t)(pos0 + t),", "(uint32_t)(b), (uint32_t)(pos0 + t),"),
    "draft_q_cumulative": ("*q = p[j];", "*q = cdf[j] / Z;"),
    "entropy_sign": ("if (p[j] > 0.0) H -= p[j] * log(p[j]);", "if (p[j] > 0.0) H += p[j] * log(p[j]);"),
    "entropy_base2": ("if (p[j] > 0.0) H -= p[j] * log(p[j]);", "if (p[j] > 0.0) H -= p[j] * log2(p[j]);"),
    "overlap_max": ("for (int64_t j = 0; j < V; ++j) s += fmin(p[j], q[j]);", "for (int64_t j = 0; j < V; ++j) s += fmax(p[j], q[j]);"),
    "overlap_next_row": ("row_ptr(target, dtype, b * (gamma + 1) + i, V)", "row_ptr(target, dtype, b * (gamma + 1) + i + 1, V)"),
    "tree_last_tie": ("if (score > best_score) {", "if (score >= best_score) {"),
    "tree_threshold_inclusive": ("if (best_score < threshold) break;", "if (best_score <= threshold) break;"),
    "tree_child_row": ("const void* trow = row_ptr(target, dtype, b * N + v, V);",
                       "const void* trow = row_ptr(target, dtype, b * N + (v + 1 < N ? v + 1 : v), V);"),
    "tree_target_only": ("else score = fmin(1.0, pp / qq);", "else score = fmin(1.0, pp);"),
    "max_ignores_first": ("for (int64_t j = 0; j < V; ++j) {\n        double l = widen(row, dtype, j);\n        if (isnan(l) || l == INFINITY) usable = 0;\n        if (l > mx) mx = l;",
                          "for (int64_t j = 1; j < V; ++j) {\n        double l = widen(row, dtype, j);\n        if (isnan(l) || l == INFINITY) usable = 0;\n        if (l > mx) mx = l;"),
}


# The pins each planted mistake fails (found by running the whole pin suite
# on every mutant); running these alone keeps the check quick, and a failure
# among them is a failure of the suite.
CATCHING_PINS = {
    "accept_flip": ['test_bonus_row_checked_only_when_reached', 'test_identical_models_accept_everything', 'test_residual_sampler_grid_mass', 'test_single_token_vocabulary', 'test_theorem_exact_enumeration_v4', 'test_tree_chain_equals_linear_verification', 'test_worked_example_exercise2'],
    "bonus_from_wrong_row": ['test_theorem_exact_enumeration_v4'],
    "draft_position": ['test_draft_cdf_interval_holds_u', 'test_draft_counters_split_across_calls', 'test_draft_uniform_row_is_floor_uV'],
    "draft_purpose": ['test_draft_cdf_interval_holds_u', 'test_draft_two_token_closed_form', 'test_draft_uniform_row_is_floor_uV'],
    "draft_q_cumulative": ['test_draft_cdf_interval_holds_u', 'test_draft_two_token_closed_form', 'test_draft_uniform_row_is_floor_uV', 'test_draft_unusable_and_masked_rows'],
    "draft_sequence": ['test_draft_cdf_interval_holds_u', 'test_draft_counters_split_across_calls', 'test_draft_uniform_row_is_floor_uV'],
    "entropy_base2": ['test_entropy_matches_scipy', 'test_entropy_of_equal_logits_is_log_V', 'test_entropy_special_rows'],
    "entropy_sign": ['test_entropy_matches_scipy', 'test_entropy_of_equal_logits_is_log_V', 'test_entropy_special_rows'],
    "greedy_last_tie": ['test_draft_greedy_is_first_argmax', 'test_greedy_matches_argmax'],
    "max_ignores_first": ['test_draft_uniform_row_is_floor_uV', 'test_entropy_of_equal_logits_is_log_V', 'test_entropy_special_rows', 'test_single_token_vocabulary', 'test_softmax_matches_library', 'test_tree_invalid_inputs'],
    "no_early_stop": ['test_invalid_inputs_positional_rule'],
    "overlap_max": ['test_expected_accept_special_cases_and_lemma1', 'test_expected_accept_worked_example'],
    "overlap_next_row": ['test_expected_accept_special_cases_and_lemma1'],
    "philox_weyl": ['test_philox_matches_aten_engine'],
    "ratio_inverted": ['test_residual_sampler_grid_mass', 'test_theorem_exact_enumeration_v4', 'test_tree_chain_equals_linear_verification', 'test_worked_example_exercise2'],
    "residual_sign": ['test_masked_draft_token_is_rejected', 'test_residual_sampler_grid_mass', 'test_theorem_exact_enumeration_v4', 'test_worked_example_exercise2'],
    "row_off_by_one": ['test_bonus_row_checked_only_when_reached', 'test_identical_models_accept_everything', 'test_invalid_inputs_positional_rule', 'test_theorem_exact_enumeration_v4', 'test_tree_chain_equals_linear_verification'],
    "sample_uses_accept_uniform": ['test_theorem_chi_square_v16'],
    "temperature_dropped": ['test_draft_two_token_closed_form', 'test_entropy_matches_scipy', 'test_entropy_special_rows', 'test_expected_accept_special_cases_and_lemma1', 'test_softmax_matches_library', 'test_theorem_exact_enumeration_v4'],
    "tree_child_row": ['test_tree_chain_equals_linear_verification', 'test_tree_greedy_follows_argmax_and_zero_threshold_reaches_a_leaf', 'test_tree_hand_example', 'test_tree_hand_example_greedy_and_ties', 'test_tree_invalid_inputs'],
    "tree_last_tie": ['test_tree_hand_example_greedy_and_ties'],
    "tree_target_only": ['test_tree_chain_equals_linear_verification', 'test_tree_hand_example', 'test_tree_hand_example_greedy_and_ties', 'test_tree_invalid_inputs'],
    "tree_threshold_inclusive": ['test_tree_hand_example'],
    "uniform_words": ['test_uniform_is_53_bit_from_words_x0_x1'],
}


def test_every_mutant_has_catching_pins():
    assert sorted(CATCHING_PINS) == sorted(MUTANTS)
    src = open(os.path.join(HERE, "test_oracle_pins.py")).read()
    for pins in CATCHING_PINS.values():
        assert pins and all(f"def {t}(" in src for t in pins)


def _run_mutant(name, workdir):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    if src.count(old) != 1:
        return None, f"mutation site for {name} not found exactly once"
    d = os.path.join(workdir, name)
    os.makedirs(d, exist_ok=True)
    mut = os.path.join(d, "oracle_mut.c")
    open(mut, "w").write(src.replace(old, new))
    so = os.path.join(d, "liboracle_mut.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-I",
                    os.path.join(ROOT, "oracle"), "-o", so, mut, "-lm"], check=True)
    env = dict(os.environ, SPECVERIFY_ORACLE_LIB=so, OMP_NUM_THREADS="2")
    pins = os.path.join(HERE, "test_oracle_pins.py")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", pins,
                        "-k", " or ".join(CATCHING_PINS[name])],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout


@pytest.fixture(scope="module")
def mutant_runs(tmp_path_factory):
    """Every mutant built and run against its pins, a few at a time."""
    from concurrent.futures import ThreadPoolExecutor
    workdir = str(tmp_path_factory.mktemp("mutants"))
    with ThreadPoolExecutor(max_workers=max(1, min(6, (os.cpu_count() or 2) - 1))) as ex:
        futs = {name: ex.submit(_run_mutant, name, workdir) for name in sorted(MUTANTS)}
        return {name: f.result() for name, f in futs.items()}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, mutant_runs):
    rc, out = mutant_runs[name]
    assert rc is not None, out
    assert rc != 0, f"mutant {name} passed every pin:\n{out[-2000:]}"
    assert "failed" in out, out[-2000:]
