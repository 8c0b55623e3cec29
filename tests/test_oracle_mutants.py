"""The oracle's pins catch plausible mistakes (mutation test, CPU only).

Each mutant is a copy of the oracle source with one plausible slip planted in it (a
transposed operand, a wrong sign, a dropped term, an off-by-one row, a reused coin,
...), at every place the statement occurs.  It is compiled into a temporary directory and swapped in for the real library;
at least one pin from the law, closed-form, special-case or golden tests must then fail.
The real oracle is restored afterwards.
"""
from __future__ import annotations

import os
import subprocess

import pytest

import oracle

import test_golden_cases as golden
import test_oracle_law as law
import test_oracle_tree_greedy as tg
import test_oracle_tree_mask as tm
import test_oracle_commit_kv as ck
import test_oracle_filtered as tf
import test_oracle_mss as ms
import test_oracle_margins as mg

SRC = open(oracle.SRC).read()

# (name, original text, planted mistake)
MUTANTS = [
    ("ratio transposed", "double ratio = p / qx;", "double ratio = qx / p;"),
    ("residual sign flipped", "double d = p - (double)q[(size_t)k * V + (size_t)x];",
     "double d = (double)q[(size_t)k * V + (size_t)x] - p;"),
    ("residual replaced by p", "w[x] = d > 0.0 ? d : 0.0;", "w[x] = p; (void)d;"),
    ("final draw from the row before",
     "Row rk = row_of(logits, dtype, b * (size_t)R + (size_t)k, V);",
     "Row rk = row_of(logits, dtype, b * (size_t)R + (size_t)(k > 0 ? k - 1 : 0), V);"),
    ("rejection coin reused for the draw", "int y = draw_inverse_cdf(w, V, (double)coins[G], margin);",
     "int y = draw_inverse_cdf(w, V, (double)coins[k], margin);"),
    ("temperature ignored", "for (int x = 0; x < r.V; ++x) Z += exp((logit(r, x) - m) / T);",
     "for (int x = 0; x < r.V; ++x) Z += exp((logit(r, x) - m));"),
    ("partition misses token 0", "for (int x = 0; x < r.V; ++x) Z += exp(",
     "for (int x = 1; x < r.V; ++x) Z += exp("),
    ("argmax ties to highest id", "if (logit(r, x) > logit(r, best)) best = x;",
     "if (logit(r, x) >= logit(r, best)) best = x;"),
    ("greedy emits the draft at the mismatch", "    out[k] = a;\n",
     "    out[k] = k < G ? draft[k] : a;\n"),
    ("bucket edge exclusive", "if (t <= C) {", "if (t < C) {"),
    ("tree prob_acc not accumulated", "acc += pc;", "acc = pc;"),
    ("tree exclusions dropped", "for (int e = 0; e < nexcl; ++e) w[excl[e]] = 0.0;", ""),
    ("tree coin of level 0 reused", "double u = (double)coins[d];", "double u = (double)coins[0];"),
    ("tree greedy follows first child", "par[c] == cur && tok[c] == a", "par[c] == cur"),
    ("accept test on q instead of p", "accept = p > 0.0 && u <= ratio;", "accept = u <= qx;"),
    ("tree mask without the node itself", "for (int j = i; j >= 0; j = par[j]) {",
     "for (int j = par[i]; j >= 0; j = par[j]) {"),
    ("tree mask transposed", "mask[(size_t)i * W + (size_t)(j / 32)] |= 1u << (j % 32);",
     "mask[(size_t)j * W + (size_t)(i / 32)] |= 1u << (i % 32);"),
    ("tree mask positions without the base", "if (pos) pos[i] = base + steps - 1;",
     "if (pos) pos[i] = steps - 1;"),
    ("tree mask positions count the node twice", "if (pos) pos[i] = base + steps - 1;",
     "if (pos) pos[i] = base + steps;"),
    ("tree mask stops below the root", "for (int j = i; j >= 0; j = par[j]) {",
     "for (int j = i; j > 0; j = par[j]) {"),
    ("commit takes the node of the same index", "if (valid && d <= k) node = d == 0 ? 0 : nodes[d - 1];",
     "if (valid && d <= k) node = d == 0 ? 0 : nodes[d < k ? d : d - 1];"),
    ("top-k keeps one token too many", "double th = tmp[top_k - 1];",
     "double th = tmp[top_k < V - 1 ? top_k : top_k - 1];"),
    ("draft row left unfiltered",
     "double Zq = filter_row(rq, mq[i], T, top_k, tp, wq, tmp, margin);",
     "double Zq = filter_row(rq, mq[i], T, 0, 1.0, wq, tmp, margin);"),
    ("target filter skipped in the acceptance test",
     "double Zp = filter_row(r, m[i], T, top_k, tp, wp, tmp, margin);",
     "double Zp = filter_row(r, m[i], T, 0, 1.0, wp, tmp, margin);"),
    ("top-p threshold one token late", "                tau = tmp[i];\n                break;",
     "                tau = tmp[i + 1 < V ? i + 1 : i];\n                break;"),
    ("commit drops the root row", "if (valid && d <= k) node = d == 0 ? 0 : nodes[d - 1];",
     "if (valid && d <= k) node = d == 0 ? -1 : nodes[d - 1];"),
    ("commit writes one row past the path", "if (valid && d <= k) node = d == 0 ? 0 : nodes[d - 1];",
     "if (valid && d <= k + 1 && d <= D) node = d == 0 ? 0 : nodes[d - 1 < D ? d - 1 : 0];"),
    ("MSS residual sign flipped", "double dv = w[v] - (double)qc[v];",
     "double dv = (double)qc[v] - w[v];"),
    ("MSS residual not renormalised", "for (int v = 0; v < V; ++v) w[v] /= S;", ""),
    ("MSS siblings tested against the original row", "double ratio = w[x] / qx;",
     "double ratio = row_prob(r, x, m, Z, T) / qx;"),
    ("MSS one coin for every sibling", "double u = (double)coins[c - 1];",
     "double u = (double)coins[0];"),
    ("MSS final draw from the target row",
     "int y = draw_inverse_cdf(w, V, (double)coins[N - 1], margin);",
     "for (int v = 0; v < V; ++v) w[v] = row_prob(r, v, m, Z, T);\n"
     "    int y = draw_inverse_cdf(w, V, (double)coins[N - 1], margin);"),
    # the near-tie margins and the acceptance-rate diagnostic
    ("draw margin in coin units", "                note_margin(mm, t - before);\n"
     "                note_margin(mm, C - t);",
     "                note_margin(mm, (t - before) / S);\n"
     "                note_margin(mm, (C - t) / S);"),
    ("draw margin dropped", "                note_margin(mm, t - before);\n"
     "                note_margin(mm, C - t);", ""),
    ("draw margin on one side only", "                note_margin(mm, C - t);\n", ""),
    ("acceptance margin against p instead of p/q", "note_margin(margin, fabs(u - ratio));",
     "note_margin(margin, fabs(u - ratio * qx));"),
    ("acceptance margin dropped", "note_margin(margin, fabs(u - ratio));", ""),
    ("residual mass not a margin", "    if (k < G) note_margin(margin, S);\n", ""),
    ("tree sibling margin dropped", "note_margin(margin, fabs(u - acc / th_acc));", ""),
    ("tree single-threshold margin dropped", "note_margin(margin, fabs(pc - th_single));", ""),
    ("accept margin includes the draw",
     "    if (amargin) *amargin = *margin; /* every margin so far: the tests before the draw */\n"
     "    if (!(S > 0.0))\n        for (int x = 0; x < V; ++x) w[x] = row_prob(rk, x, m[k], Z[k], T);\n"
     "    int y = draw_inverse_cdf(w, V, (double)coins[G], margin);\n",
     "    if (!(S > 0.0))\n        for (int x = 0; x < V; ++x) w[x] = row_prob(rk, x, m[k], Z[k], T);\n"
     "    int y = draw_inverse_cdf(w, V, (double)coins[G], margin);\n"
     "    if (amargin) *amargin = *margin;\n"),
    ("beta sums the larger of p and q", "s += p < qq ? p : qq;", "s += p > qq ? p : qq;"),
    ("beta from the next row", "Row r = row_of(logits, dtype, b * (size_t)R + (size_t)i, V);\n"
     "            double mi = row_max(r);",
     "Row r = row_of(logits, dtype, b * (size_t)R + (size_t)(i + 1), V);\n"
     "            double mi = row_max(r);"),
]


def _pins():
    """Callables that raise AssertionError when a pin fails."""
    yield lambda: law.test_chain_round_emits_target_law(0, 0.0, 1.0)
    yield lambda: law.test_chain_round_emits_target_law(2, 0.0, 0.7)
    yield law.test_chain_acceptance_rate_and_residual_law
    yield lambda: law.test_expected_tokens_closed_form(22, 3)
    yield lambda: law.test_probs_match_scipy_softmax("bf16", 0.7)
    yield law.test_bonus_draw_is_inverse_cdf
    yield law.test_degenerate_p_q_cases
    yield lambda: tg.test_greedy_chain_equals_autoregressive(1, 4, 0.7)
    yield tg.test_greedy_ties_go_to_lowest_id
    yield tg.test_greedy_tree_equals_autoregressive
    yield lambda: tg.test_tree_walk_emits_target_law(0, 1.0)
    yield lambda: tg.test_tree_walk_emits_target_law(1, 1.0)
    yield tg.test_tree_rejected_children_are_removed_from_final_draw
    for case in golden.CASES["chain"]:
        yield lambda case=case: golden.test_chain_hand_case(case)
    for case in golden.CASES["tree"]:
        yield lambda case=case: golden.test_tree_hand_case(case)
    yield lambda: tm.test_chain_is_lower_triangular(33)
    yield tm.test_golden_cases
    yield lambda: tm.test_masked_tree_attention_equals_per_branch_causal_attention(0)
    yield lambda: ck.test_committed_rows_equal_sequential_decode_of_the_emitted_prefix(
        oracle.TREE_SAMPLING, 0)
    yield ck.test_chain_shaped_tree_commits_in_place_order
    yield tf.test_top1_is_greedy_verify
    for case in tf.GOLDEN["cases"]:
        yield lambda case=case: tf.test_golden(case)
    yield lambda: tf.test_filtered_round_emits_filtered_target_law(2, 4, 0.8, 0.7)
    yield ms.test_hand_first_child_accepted
    yield ms.test_hand_second_child_accepted_after_residual
    yield ms.test_hand_both_rejected_final_draw_from_residual
    yield lambda: ms.test_chain_shaped_tree_equals_chain_verify(0, 1.0)
    yield lambda: ms.test_walk_emits_target_law_over_coins_and_drafts(0, 1.0, [-1, 0, 0, 1, 1, 2])
    yield lambda: mg.test_chain_margins_equal_breakpoint_distances(0, 1.0)
    yield mg.test_chain_margin_is_small_exactly_when_a_nudge_flips_the_result
    yield lambda: mg.test_beta_equals_lattice_acceptance_rate(0)
    yield lambda: mg.test_tree_margins_equal_breakpoint_distances(0, 1.5)
    yield lambda: mg.test_tree_margins_equal_breakpoint_distances(2, 6.0)


@pytest.mark.parametrize("name,orig,mutation", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, orig, mutation, tmp_path):
    assert SRC.count(orig) >= 1, f"mutation anchor not found: {orig}"
    src = tmp_path / "spec_oracle.c"
    src.write_text(SRC.replace(orig, mutation))
    hdr = os.path.join(os.path.dirname(oracle.SRC), "spec_oracle.h")
    (tmp_path / "spec_oracle.h").write_text(open(hdr).read())
    so = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                    "-w", "-o", str(so), str(src), "-lm"], check=True)
    saved_lib, saved_path = oracle._lib, oracle.LIB_PATH
    try:
        oracle._lib = None
        oracle.LIB_PATH = str(so)
        caught = []
        for pin in _pins():
            try:
                pin()
            except (AssertionError, ValueError):
                caught.append(pin)
                break
        assert caught, f"no pin caught mutant '{name}'"
    finally:
        oracle._lib, oracle.LIB_PATH = saved_lib, saved_path
