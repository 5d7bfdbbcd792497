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


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-I",
                    os.path.join(ROOT, "oracle"), "-o", str(so), str(mut), "-lm"], check=True)
    env = dict(os.environ, SPECVERIFY_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout, r.stdout[-2000:]
