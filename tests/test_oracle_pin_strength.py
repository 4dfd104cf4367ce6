"""Pin strength: plausible mistakes planted in the oracle are caught.

Each case below copies one oracle function, changes one expression in the
copy (a dropped term, a wrong sign, an off-by-one, a transposed index, the
wrong tie order or rounding), installs the copy in place of the original
for the duration of the case, and runs the pins that guard that function.
At least one pin must fail.  Everything runs on the CPU; nothing here
touches the GPU path.
"""
import inspect
import textwrap

import pytest

from oracle import materialise, numerics, paging, rope, score, select

import test_oracle_actkv_policy as T_act
import test_oracle_numerics_paging as T_num
import test_oracle_rope_materialise as T_rm
import test_oracle_score as T_sc
import test_oracle_select as T_sel


def _mutant(fn, old, new):
    src = textwrap.dedent(inspect.getsource(fn))
    assert src.count(old) == 1, "the planted change must match exactly once: %r" % old
    g = dict(fn.__globals__)
    exec(compile(src.replace(old, new), "<planted %s>" % fn.__name__, "exec"), g)
    return g[fn.__name__]


# (module, function, expression, planted replacement, pins that guard it)
CASES = [
    # window scores
    ("score", "window_scores", "np.arange(N)[None, :] <= pos[:, None]", "np.arange(N)[None, :] < pos[:, None]",
     [T_sc.test_causal_window_rows_see_only_their_prefix, T_sc.test_softmax_rows_sum_to_one_and_totals_equal_row_count]),
    ("score", "window_scores", "np.exp(s - lse[..., None])", "np.exp(lse[..., None] - s)",
     [T_sc.test_two_key_closed_form_fixes_scale]),
    ("score", "window_scores", "scale = 1.0 / np.sqrt(D)", "scale = 1.0 / D",
     [T_sc.test_two_key_closed_form_fixes_scale]),
    ("score", "window_scores", "if gqa_group(h, Hq, Hkv) == g]", "if h % Hkv == g]",
     [T_sc.test_gqa_groups_are_consecutive_query_heads]),
    ("score", "window_scores", 'scores[l, g] = _reduce(_reduce(p, head_agg, 0), row_agg, 0)',
     'scores[l, g] = _reduce(_reduce(p, row_agg, 1), head_agg, 0)',
     [T_sc.test_max_over_group_then_mean_over_rows]),
    # pooling
    ("score", "pool1d", "out[..., ok] += a[..., src[ok]]", "out[..., ok] += a[..., idx[ok]]",
     [lambda: T_sc.test_pool_impulse_response(5), T_sc.test_pool_avg_total_is_coverage_weighted]),
    ("score", "pool1d", "out[..., ok] = np.maximum(out[..., ok], a[..., src[ok]])",
     "out[..., ok] = np.maximum(out[..., ok], a[..., idx[ok]])",
     [lambda: T_sc.test_pool_impulse_response(5)]),
    # session memory
    ("score", "memory_update", "m = decay * m_prev + e", "m = decay * m_prev + (1 - decay) * e",
     [T_sc.test_memory_two_turn_closed_form]),
    ("score", "memory_scores", "lse = _logsumexp(s, H)", "lse = _logsumexp(s, np.ones_like(H))",
     [T_sc.test_memory_scores_history_excludes_forced_and_dead]),
    ("score", "memory_scores", "g = gqa_group(h, Hq, Hkv)", "g = h % Hkv",
     [T_sc.test_memory_scores_equal_single_row_window_scores]),
    # block scores and the Mean-K index
    ("score", "block_scores", "scale = 1.0 / np.sqrt(D)", "scale = 1.0 / D",
     [T_sc.test_block_score_hand_example, T_sc.test_block_scores_equal_per_query_brute_force]),
    ("score", "query_reduce", "q[:, :, h].sum(axis=2)", "q[:, :, h].mean(axis=2)",
     [T_sc.test_block_scores_equal_per_query_brute_force]),
    ("score", "mean_k_index", "numerics.round_to_f16(blocks.sum(axis=-2) / bt)",
     "numerics.round_to_bf16(blocks.sum(axis=-2) / bt)",
     [T_sc.test_mean_k_rounds_once_to_float16_nearest_even, T_sc.test_mean_k_hand_example_two_blocks]),
    ("score", "mean_k_index", "reshape(*lead, nb, bt, d)", "reshape(*lead, bt, nb, d).swapaxes(-3, -2)",
     [T_sc.test_mean_k_hand_example_two_blocks]),
    # the decode-streaming action scorer
    ("score", "decode_recovery_step", "np.max(np.stack(probs), axis=0)", "np.sum(np.stack(probs), axis=0)",
     [lambda: T_act.test_running_mean_equals_batch_window_mean(2), T_act.test_two_token_hand_example]),
    ("score", "decode_recovery_step", "(p - st[l, r, g]) / (t + 1)", "(p - st[l, r, g]) / t",
     [T_act.test_two_token_hand_example]),
    ("score", "decode_recovery_step", "visible = (j < n)", "visible = (j <= n)",
     [lambda: T_act.test_running_mean_equals_batch_window_mean(1)]),
    ("score", "decode_recovery_step", "@ q[l, a, h]) - lse[l, a, h])", "@ q[l, a, h]) + lse[l, a, h])",
     [T_act.test_lse_identity_single_head_sums_to_one]),
    ("score", "decode_recovery_step", "if t == 0:", "if t < 0:",
     [T_act.test_region_start_discards_old_state_and_inactive_requests_stay]),
    # selection
    ("select", "select_topk", "order = np.lexsort((cand, -s[cand]))", "order = np.lexsort((-cand, -s[cand]))",
     [T_sel.test_negative_zero_ties_positive_zero, T_sel.test_topk_equals_max_sum_brute_force]),
    ("select", "select_topk", "room = k_total - int(f.sum())", "room = k_total - n_sink - n_recent",
     [T_sel.test_invariants_on_random_units]),
    ("select", "select_topk_tiled", "run_idx = pool[order[:room]]", "run_idx = pool[order[:room - 1]]",
     [T_sel.test_tiled_equals_untiled]),
    # top-p hits and the LRFU keep score
    ("select", "top_p_hits", 'side="left"', 'side="right"', [T_act.test_top_p_hand_examples]),
    ("select", "top_p_hits", "order = np.lexsort((np.arange(n), -s))", "order = np.lexsort((-np.arange(n), -s))",
     [T_act.test_top_p_hand_examples]),
    ("select", "top_p_hits", "cum = np.cumsum(s[order])", "cum = np.cumsum(s[order]) - s[order]",
     [T_act.test_top_p_is_a_minimum_cardinality_set_by_brute_force]),
    ("select", "lrfu_keep_score", "return lam * ks +", "return (1.0 - lam) * ks +", [T_act.test_lambda_limits]),
    ("select", "lrfu_keep_score", "np.where(hits, np.asarray(scores, dtype=np.float64), 0.0)",
     "np.asarray(scores, dtype=np.float64)", [T_act.test_lambda_limits]),
    # the decay dropped: hits accumulate at every lambda
    ("select", "lrfu_keep_score", "return lam * ks +", "return ks +",
     [T_act.test_intermediate_lambda_behaviour_the_page_describes]),
    ("select", "action_scores", "math.fsum(st[:, :, j].reshape(L * Hkv).tolist())", "float(np.max(st[:, :, j]))",
     [T_act.test_action_scores_sum_units_exactly_then_round_to_f32]),
    # RoPE
    ("rope", "rope_rotate", "out[..., :half] = a * c - b * s", "out[..., :half] = a * c + b * s",
     [T_rm.test_rope_d2_theta1_is_rotation_by_p_radians]),
    ("rope", "inv_freq", "-2.0 * m / rotary_dim", "-1.0 * m / rotary_dim",
     [T_rm.test_rope_pairs_and_frequencies_d4]),
    # materialisation
    ("materialise", "gather_view", "rope_rotate(k_out, p_new - rows,", "rope_rotate(k_out, p_new + rows,",
     [T_rm.test_gather_delta_on_baked_matches_raw_within_two_ulp]),
    ("materialise", "gather_view", "rows = (idx[:, None] * bt + np.arange(bt)[None, :])",
     "rows = (idx[:, None] + np.arange(bt)[None, :])", [T_rm.test_gather_plain_copies_bit_for_bit]),
    ("materialise", "incremental_view", "delta = (i_new - i_old) * bt", "delta = (i_old - i_new) * bt",
     [lambda: T_rm.test_incremental_equals_fresh_build(40)]),
    ("materialise", "redirect", "np.where(np.asarray(keep_mask, dtype=bool), sm, dead_slot)",
     "np.where(~np.asarray(keep_mask, dtype=bool), sm, dead_slot)", [T_rm.test_redirect_invariants]),
    ("materialise", "free_list", " or u in kept_slots:", ":",
     [T_rm.test_free_list_hand_example, T_rm.test_reusing_freed_slots_never_changes_a_kept_or_sibling_read]),
    ("materialise", "free_list", "j < protected_len", "j <= protected_len", [T_rm.test_free_list_hand_example]),
    ("materialise", "tail_compact", "X = -(-n_kept // bs)", "X = n_kept // bs",
     [T_rm.test_tail_compact_hand_example, lambda: T_rm.test_tail_compact_preserves_kept_entries(0)]),
    ("materialise", "tail_compact", "zip(sources, dests)", "zip(sources, dests[::-1])",
     [T_rm.test_tail_compact_hand_example]),
    # shared helpers and the remaining steps
    ("score", "gqa_group", "return h // (n_q_heads // n_kv_heads)", "return h % n_kv_heads",
     [T_sc.test_gqa_groups_are_consecutive_query_heads]),
    ("score", "_logsumexp", "return (m_safe + np.log(tot))[..., 0]", "return np.log(tot)[..., 0]",
     [T_sc.test_two_key_closed_form_fixes_scale, T_sc.test_softmax_rows_sum_to_one_and_totals_equal_row_count]),
    ("score", "history_mask", "(j >= n - n_recent)", "(j > n - n_recent)",
     [T_sc.test_memory_scores_history_excludes_forced_and_dead]),
    ("select", "forced_mask", "(j >= n - n_recent)", "(j > n - n_recent)",
     [T_sel.test_budget_edge_cases, T_sel.test_topk_equals_max_sum_brute_force]),
    ("select", "keep_score_step", "n = int(n_len[r])", "n = n_cap",
     [T_act.test_keep_score_step_per_request]),
    ("materialise", "decode_attention_slots", "s = (K @ q) * scale", "s = (K @ q)",
     [T_rm.test_decode_attention_two_key_closed_form]),
    ("materialise", "sentinel_rows", "np.full(D, -1.0e4)", "np.full(D, -1.0e3)",
     [T_num.test_sentinel_bits_match_fixture]),
    ("paging", "logical_keys_from_pool", "return np.transpose(rows, (1, 0, 2))",
     "return rows.reshape(rows.shape[1], rows.shape[0], rows.shape[2])", [T_num.test_logical_keys_through_pages]),
    # paging and rounding
    ("paging", "slot_map_from_block_table", "bt[j // block_size] * block_size + j % block_size",
     "bt[j % block_size] * block_size + j // block_size", [T_num.test_slot_map_worked_example]),
    ("numerics", "_round_sig", "r = np.rint(xf / q) * q", "r = np.floor(xf / q + 0.5) * q",
     [T_num.test_bf16_halfway_cases_round_to_even]),
    ("numerics", "round_to_f16", "_round_sig(x, 11, -24, 65520.0)", "_round_sig(x, 10, -24, 65520.0)",
     [T_num.test_f16_matches_numpy_half]),
]

MODULES = {"score": score, "select": select, "rope": rope, "materialise": materialise, "paging": paging,
           "numerics": numerics}


@pytest.mark.parametrize("case", CASES, ids=["%s.%s:%s" % (c[0], c[1], c[3][:40]) for c in CASES])
def test_planted_mistake_is_caught(case, monkeypatch):
    mod_name, fn_name, old, new, pins = case
    original = getattr(MODULES[mod_name], fn_name)
    planted = _mutant(original, old, new)
    # replace every binding of the function, including names imported into
    # other oracle modules and into the pin modules
    for m in list(MODULES.values()) + [T_act, T_num, T_rm, T_sc, T_sel]:
        if getattr(m, fn_name, None) is original:
            monkeypatch.setattr(m, fn_name, planted)
    for pin in pins:
        try:
            pin()
        except AssertionError:
            return
    pytest.fail("no pin caught %s.%s with %r -> %r" % (mod_name, fn_name, old, new))

