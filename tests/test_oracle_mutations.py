"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case rewrites one expression of an oracle function's source (a dropped
term, a flipped sign or comparison, an off-by-one, a transposed operand),
installs the mutant in place of the original for the duration of the test and
checks that at least one of the pins fails.  This shows the pins are strong
enough to catch plausible mistakes, not only that the oracle passes them.
"""
import inspect
import textwrap

import pytest

import oracle.dense as dense
import oracle.fidelity as fid
import oracle.kap as kap
import oracle.osk as osk
import tests.test_oracle_dense as td
import tests.test_oracle_fidelity as tf
import tests.test_oracle_kap as tk
import tests.test_oracle_osk as to


def _mutant(module, fname, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(module, fname)))
    assert old in src, f"mutation anchor {old!r} not found in {fname}"
    ns = dict(module.__dict__)
    exec(compile(src.replace(old, new, 1), f"<mutant {fname}>", "exec"), ns)
    return ns[fname]


def _fails(*checks):
    for c in checks:
        try:
            c()
        except Exception:   # a failed assertion or a crash both reveal the mutant
            return True
    return False


MUTATIONS = [
    # dense: causal mask off by one (strictly-before keys only)
    (dense, "attention_rows", "<= row_pos[:, None]", "< row_pos[:, None]",
     [td.test_zero_queries_give_running_mean_of_values]),
    # dense: transposed key operand in the logits (q @ k instead of q @ k.T) on square input
    (dense, "attention_rows", "q_rows @ k.T", "(q_rows @ k.T).T",
     [td.test_dense_matches_torch_sdpa_fp64_gqa]),
    # dense: scale dropped
    (dense, "attention_rows", "s = scale * (q_rows @ k.T)", "s = (q_rows @ k.T)",
     [td.test_dense_matches_torch_sdpa_fp64_gqa]),
    # KAP: score sorted ascending instead of descending
    (kap, "flag_grouped_order", "(j, -w, (~hrm)", "(j, w, (~hrm)",
     [lambda: tk.test_golden_worked_example(0), lambda: tk.test_golden_worked_example(1)]),
    # KAP: HRM group placed last
    (kap, "flag_grouped_order", "(~hrm).astype", "(hrm).astype",
     [lambda: tk.test_golden_worked_example(0)]),
    # KAP: tie-break by descending block index
    (kap, "flag_grouped_order", "np.lexsort((j,", "np.lexsort((-j,",
     [lambda: tk.test_golden_worked_example(1)]),
    # KAP: ceil replaced by floor in the budget count
    (kap, "budget_count", "+ 999_999", "+ 0",
     [tk.test_budget_counts_hand_values]),
    # KAP: importance averaged over all R rows ignoring candidacy (drops the softmax normalisation)
    (kap, "score_tile", "p = e / e.sum(axis=1, keepdims=True)", "p = e",
     [lambda: tk.test_golden_worked_example(0)]),
    # KAP: proxy-row candidates off by one block
    (kap, "score_tile", "<= (last // kv_block)[:, None]", "< (last // kv_block)[:, None]",
     [lambda: tk.test_golden_worked_example(0)]),
    # OSK: skip comparison flipped
    (osk, "osk_tile_sequential", "np.all(bm < m - tau)", "np.all(bm > m - tau)",
     [to.test_skip_rule_hand_example]),
    # OSK: skip decided with any() instead of the per-row AND
    (osk, "osk_tile_sequential", "np.all(bm < m - tau)", "np.any(bm < m - tau)",
     [to.test_bucket_effect_one_row_vetoes]),
    # OSK: rescale factor dropped from the accumulator
    (osk, "osk_tile_sequential", "o = alpha[:, None] * o + p @ v[a:e]", "o = o + p @ v[a:e]",
     [to.test_order_invariance_without_skip, to.test_full_budget_no_skip_equals_dense_ragged]),
    # OSK: skip threshold with the wrong sign of tau
    (osk, "osk_tile_sequential", "np.all(bm < m - tau)", "np.all(bm < m + tau)",
     [to.test_skip_rule_hand_example]),
    # Top-p: mass accumulated in plain score order instead of the HRM-first order
    (kap, "kap_tile", "top_p_count(w[order], top_p)", "top_p_count(np.sort(w)[::-1], top_p)",
     [lambda: tk.test_top_p_golden(2)]),
    # Top-p: reaching p exactly not counted as reached
    (kap, "top_p_count", "np.cumsum(w_in_order) >= p", "np.cumsum(w_in_order) > p",
     [tk.test_top_p_count_hand_values]),
    # Top-p: off by one (the block that crosses p left out)
    (kap, "top_p_count", "int(reached[0]) + 1", "max(int(reached[0]), 1)",
     [lambda: tk.test_top_p_golden(1), tk.test_top_p_count_hand_values]),
    # Top-p: budget cap ignored
    (kap, "kap_tile", "k = min(k, top_p_count(", "k = (0 * k + top_p_count(",
     [lambda: tk.test_top_p_golden(5)]),
    # Delta / N: threshold inverted to ln(Delta / N)
    (osk, "tau_from_delta", "math.log(seqlen / delta)", "math.log(delta / seqlen)",
     [to.test_tau_from_delta_hand_values]),
    # GQA-shared mask: only the first head's proxy rows scored
    (kap, "group_tiles", "for qb, _, va in pooled]", "for qb, _, va in pooled[:1]]",
     [tk.test_gqa_shared_golden]),
    # fidelity: exact top-k picks the smallest masses
    (fid, "top_mass_blocks", "-mass))", "mass))",
     [tf.test_top_mass_and_iou_hand_values]),
    # fidelity: the diagonal key dropped from the exact mass
    (fid, "exact_block_mass", "<= row_pos[:, None]", "< row_pos[:, None]",
     [tf.test_uniform_attention_block_mass_by_hand]),
    # Delta / N: skip switched off whenever tau_b comes out negative
    (osk, "osk_prefill", "on = delta > 0", "on = delta > 0 and tau_from_delta(L, delta) >= 0",
     [lambda: to.test_delta_mode_negative_tau_still_skips(False)]),
]


@pytest.mark.parametrize("case", range(len(MUTATIONS)))
def test_planted_mistake_is_caught(case, monkeypatch):
    module, fname, old, new, checks = MUTATIONS[case]
    monkeypatch.setattr(module, fname, _mutant(module, fname, old, new))
    assert _fails(*checks), f"mutation {old!r} -> {new!r} in {fname} was not caught"
