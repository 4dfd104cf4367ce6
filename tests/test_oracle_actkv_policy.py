"""Pins for the oracle's decode-streaming action scorer and LRFU keep score
(CPU only).

The scorer is checked against the pinned batch window scorer (a running
mean over T decode tokens must equal the plain mean over a T-row causal
window), against the LSE identity (recovered probabilities of one head sum
to one) and against a hand-computed two-token example.  The keep score is
checked against hand-worked top-p sets, brute force over all subsets, and
the two limits (lambda = 0 and lambda = 1) that ActKV §5.2 describes.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import paging, score, select


def _rng(seed):
    return np.random.default_rng(seed)


def _paged(rng, L, R, Hkv, D, BS, n_pos):
    """A pool with every request's blocks at shuffled physical blocks."""
    Y = -(-n_pos // BS)
    P = R * Y + 3
    perm = rng.permutation(P)[: R * Y].reshape(R, Y)
    k_pool = rng.standard_normal((L, P, BS, Hkv, D))
    return k_pool, perm


# ---------------------------------------------------------------- decode scorer

@pytest.mark.parametrize("G", [1, 2, 4])
def test_running_mean_equals_batch_window_mean(G):
    # T decode tokens of one action region, context growing by one per token:
    # the streamed state equals window_scores(head_agg=max, row_agg=mean) on
    # the same keys read back in logical order through the block table
    rng = _rng(11 + G)
    L, R, Hkv, D, BS = 2, 3, 2, 8, 4
    Hq = G * Hkv
    N0, T = 9, 5
    N = N0 + T
    n_cap = N + 6
    k_pool, bt = _paged(rng, L, R, Hkv, D, BS, n_cap)
    qs = rng.standard_normal((T, L, R, Hq, D)) * 1.5
    state = np.full((L, R, Hkv, n_cap), np.nan)          # a region start never reads it
    for t in range(T):
        # the attention pass's log-sum-exp over the keys the token sees
        n_ctx = np.full(R, N0 + t + 1)
        lse = np.empty((L, R, Hq))
        for r in range(R):
            sm = paging.slot_map_from_block_table(bt[r], BS, int(n_ctx[r]))
            for l in range(L):
                k = paging.logical_keys_from_pool(k_pool[l], sm, BS)
                for h in range(Hq):
                    s = k[score.gqa_group(h, Hq, Hkv)] @ qs[t, l, r, h] / math.sqrt(D)
                    lse[l, r, h] = np.log(np.sum(np.exp(s - s.max()))) + s.max()
        state = score.decode_recovery_step(state, np.full(R, t), qs[t], lse, k_pool, bt, n_ctx)
    for r in range(R):
        sm = paging.slot_map_from_block_table(bt[r], BS, N)
        k = np.stack([paging.logical_keys_from_pool(k_pool[l], sm, BS) for l in range(L)])
        qwin = np.transpose(qs[:, :, r], (1, 2, 0, 3))                 # [L][Hq][T][D]
        want, _ = score.window_scores(qwin, k, causal=True, head_agg="max", row_agg="mean")
        np.testing.assert_allclose(state[:, r, :, :N], want, rtol=1e-12, atol=1e-15)
        assert np.all(state[:, r, :, N:] == 0.0)


def test_lse_identity_single_head_sums_to_one():
    rng = _rng(3)
    L, R, Hkv, D, BS, n = 2, 2, 3, 16, 8, 37
    k_pool, bt = _paged(rng, L, R, Hkv, D, BS, n)
    q = rng.standard_normal((L, R, Hkv, D))
    lse = np.empty((L, R, Hkv))
    for r in range(R):
        sm = paging.slot_map_from_block_table(bt[r], BS, n)
        for l in range(L):
            k = paging.logical_keys_from_pool(k_pool[l], sm, BS)
            for g in range(Hkv):
                s = k[g] @ q[l, r, g] / 4.0
                lse[l, r, g] = math.log(math.fsum(np.exp(s).tolist()))
    st = score.decode_recovery_step(np.zeros((L, R, Hkv, 40)), np.zeros(R, int), q, lse, k_pool, bt,
                                    np.full(R, n))
    np.testing.assert_allclose(st.sum(axis=3), 1.0, rtol=1e-13)


def test_two_token_hand_example():
    # D = 2, scale 1, one KV head serving two query heads, keys (0,0) and
    # (ln 3, 0) in one block of size 2.
    # token 1: head 0 q = (1,0): p = (1/4, 3/4); head 1 q = 0: p = (1/2, 1/2)
    #          max = (1/2, 3/4)
    # token 2: head 0 q = (-1,0): p = (3/4, 1/4); head 1 q = 0: (1/2, 1/2)
    #          max = (3/4, 1/2); mean of the two tokens = (5/8, 5/8)
    ln3 = math.log(3.0)
    k_pool = np.zeros((1, 2, 2, 1, 2))
    k_pool[0, 1, 1, 0, 0] = ln3              # physical block 1 holds logical block 0
    bt = np.array([[1]])
    q1 = np.array([[[[1.0, 0.0], [0.0, 0.0]]]])
    lse1 = np.array([[[math.log(4.0), math.log(2.0)]]])
    st = score.decode_recovery_step(np.zeros((1, 1, 1, 3)), [0], q1, lse1, k_pool, bt, [2], scale=1.0)
    np.testing.assert_allclose(st[0, 0, 0], [0.5, 0.75, 0.0], atol=1e-15)
    q2 = np.array([[[[-1.0, 0.0], [0.0, 0.0]]]])
    lse2 = np.array([[[math.log(4.0 / 3.0), math.log(2.0)]]])
    st = score.decode_recovery_step(st, [1], q2, lse2, k_pool, bt, [2], scale=1.0)
    np.testing.assert_allclose(st[0, 0, 0], [0.625, 0.625, 0.0], atol=1e-15)


def test_region_start_discards_old_state_and_inactive_requests_stay():
    rng = _rng(5)
    L, R, Hkv, D, BS = 1, 3, 2, 8, 4
    k_pool, bt = _paged(rng, L, R, Hkv, D, BS, 16)
    q = rng.standard_normal((L, 2, 2 * Hkv, D))
    lse = rng.standard_normal((L, 2, 2 * Hkv)) + 3.0
    old = rng.random((L, R, Hkv, 16))
    a = score.decode_recovery_step(old, [0, 0, 0], q, lse, k_pool, bt, [16, 16, 16], req=[2, 0])
    b = score.decode_recovery_step(np.zeros_like(old), [0, 0, 0], q, lse, k_pool, bt, [16, 16, 16],
                                   req=[2, 0])
    np.testing.assert_array_equal(a[:, [0, 2]], b[:, [0, 2]])
    np.testing.assert_array_equal(a[:, 1], old[:, 1])        # request 1 is not generating an action


def test_unmapped_blocks_and_unseen_positions_score_zero():
    rng = _rng(6)
    L, R, Hkv, D, BS = 1, 1, 1, 4, 4
    k_pool = rng.standard_normal((L, 3, BS, Hkv, D))
    bt = np.array([[2, 7, 0]])                 # logical block 1 points outside the pool
    q = rng.standard_normal((L, 1, 1, D))
    st = score.decode_recovery_step(np.zeros((1, 1, 1, 12)), [0], q, np.zeros((1, 1, 1)), k_pool, bt,
                                    [10])
    assert np.all(st[0, 0, 0, 4:8] == 0.0) and np.all(st[0, 0, 0, 10:] == 0.0)
    assert np.all(st[0, 0, 0, :4] > 0.0) and np.all(st[0, 0, 0, 8:10] > 0.0)


# ---------------------------------------------------------------- top-p and LRFU

def test_top_p_hand_examples():
    s = np.array([1.0, 8.0, 2.0, 5.0]) / 16
    # descending: 8, 5, 2, 1 -> cumulative 8/16, 13/16, 15/16 >= 0.9
    assert select.top_p_hits(s, 0.9).tolist() == [False, True, True, True]
    assert select.top_p_hits(s, 0.5).tolist() == [False, True, False, False]
    # equal scores: the lower index comes first
    t = np.full(4, 0.25)
    assert select.top_p_hits(t, 0.5).tolist() == [True, True, False, False]
    assert select.top_p_hits(t, 0.51).tolist() == [True, True, True, False]
    # top_p = 1: every positive entry and no zero
    u = np.array([0.0, 3.0, 0.0, 1.0])
    assert select.top_p_hits(u, 1.0).tolist() == [False, True, False, True]
    assert not select.top_p_hits(np.zeros(5), 0.9).any()
    assert select.top_p_hits(np.zeros(0), 0.9).shape == (0,)


def test_top_p_is_a_minimum_cardinality_set_by_brute_force():
    rng = _rng(9)
    for trial in range(300):
        n = int(rng.integers(1, 8))
        s = rng.integers(0, 6, size=n).astype(float) / 8.0      # exact sums, many ties
        p = float(rng.choice([0.3, 0.5, 0.9, 1.0]))
        hit = select.top_p_hits(s, p)
        target = p * s.sum()
        if target <= 0:
            assert not hit.any()
            continue
        m_best = min(m for m in range(n + 1)
                     for c in itertools.combinations(range(n), m) if s[list(c)].sum() >= target)
        assert hit.sum() == m_best
        assert s[hit].sum() >= target
        # a prefix of the order: every hit outranks every miss
        for i in np.nonzero(hit)[0]:
            for j in np.nonzero(~hit)[0]:
                assert s[i] > s[j] or (s[i] == s[j] and i < j)


def test_action_scores_sum_units_exactly_then_round_to_f32():
    st = np.zeros((2, 1, 2, 3))
    st[:, 0, :, 0] = [[0.25, 0.5], [0.125, 0.0625]]
    st[0, 0, 0, 1] = 1.0
    st[1, 0, 1, 1] = 2.0 ** -30                    # kept by the exact sum, lost by float32 rounding
    a = select.action_scores(st, 0, 3)
    assert a.tolist() == [0.9375, 1.0, 0.0]
    st[1, 0, 1, 1] = 2.0 ** -23                    # one float32 ulp of 1.0
    assert select.action_scores(st, 0, 2).tolist() == [0.9375, 1.0 + 2.0 ** -23]


def test_lambda_limits():
    rng = _rng(12)
    n, T = 20, 4
    scores = [rng.random(n) ** 3 for _ in range(T)]
    hits = [select.top_p_hits(a, 0.9) for a in scores]
    ks0 = rng.random(n)
    # lambda = 0: recency -- only the latest step counts
    k = ks0
    for a, h in zip(scores, hits):
        k = select.lrfu_keep_score(k, a, h, 0.0)
    np.testing.assert_array_equal(k, np.where(hits[-1], scores[-1], 0.0))
    # lambda = 1: frequency -- every hit accumulates, nothing decays
    k = ks0
    for a, h in zip(scores, hits):
        k = select.lrfu_keep_score(k, a, h, 1.0)
    np.testing.assert_allclose(k, ks0 + sum(np.where(h, a, 0.0) for a, h in zip(scores, hits)),
                               rtol=1e-15)
    # 0 < lambda < 1: a missed step decays the score geometrically
    k = select.lrfu_keep_score(np.array([1.0]), [0.5], [False], 0.25)
    assert k.tolist() == [0.25]


def test_intermediate_lambda_behaviour_the_page_describes():
    """ActKV §5.2 describes what each regime does to two kinds of entries: an
    intermittent entry with high attention that goes quiet for a while, and a
    continuous entry that stops being attended (stale).  At lambda = 0 the
    quiet intermittent entry falls to the bottom; at lambda = 1 the stale
    continuous entry keeps outranking a newly important one; with 0 < lambda
    < 1 the intermittent entry survives its quiet steps and the stale entry
    is overtaken.  The update equation itself is lost from the page, so this
    pins the behaviour, not the formula."""
    # entries: I (intermittent), O (continuous, stale from step 4), N (new,
    # attended from step 4), Z (never attended); scores and hits per step
    steps = [
        ([1.0, 0.4, 0.0, 0.0], [True, True, False, False]),
        ([0.01, 0.4, 0.0, 0.0], [False, True, False, False]),
        ([0.01, 0.4, 0.0, 0.0], [False, True, False, False]),
        ([0.01, 0.0, 0.5, 0.0], [False, False, True, False]),
        ([0.01, 0.0, 0.5, 0.0], [False, False, True, False]),
    ]
    I, O, N, Z = range(4)

    def run(lam, upto):
        k = np.zeros(4)
        for a, h in steps[:upto]:
            k = select.lrfu_keep_score(k, np.array(a), np.array(h), lam)
        return k

    # after its two quiet steps, the intermittent entry
    assert run(0.0, 3)[I] == run(0.0, 3)[Z] == 0.0          # lambda = 0: no better than never attended
    for lam in (0.3, 0.5, 0.7):
        k = run(lam, 3)
        assert k[I] > k[Z] and k[I] > 0.0                    # 0 < lambda < 1: it survives
    # after the new entry's two steps, the stale continuous entry
    k = run(1.0, 5)
    assert k[O] > k[N]                                       # lambda = 1: the stale entry is retained
    for lam in (0.3, 0.5, 0.7):
        k = run(lam, 5)
        assert k[N] > k[O]                                   # 0 < lambda < 1: it decays below the new one


def test_keep_score_step_per_request():
    rng = _rng(14)
    L, R, Hkv, n_cap = 2, 3, 2, 10
    state = rng.random((L, R, Hkv, n_cap)) ** 4
    ks = rng.random((R, n_cap))
    n_len = np.array([10, 7, 4])
    ks2, hit, attn = select.keep_score_step(state, ks, n_len, lam=0.5, top_p=0.9, req=[2, 1])
    np.testing.assert_array_equal(ks2[0], ks[0])                  # not compressing now
    assert not hit[0].any() and not attn[0].any()
    for r in (1, 2):
        n = n_len[r]
        a = select.action_scores(state, r, n)
        h = select.top_p_hits(a, 0.9)
        np.testing.assert_array_equal(hit[r, :n], h)
        np.testing.assert_array_equal(ks2[r, :n], 0.5 * ks[r, :n] + np.where(h, a, 0.0))
        np.testing.assert_array_equal(ks2[r, n:], ks[r, n:])
        assert not hit[r, n:].any()


def test_keep_score_step_rejects_lengths_beyond_the_row():
    # a request cannot hold more entries than its row, nor fewer than none
    state = np.ones((1, 2, 1, 5))
    ks = np.zeros((2, 5))
    for bad in (6, -1):
        with pytest.raises(ValueError):
            select.keep_score_step(state, ks, np.array([5, bad]), lam=0.5)
    # requests not listed are not read
    select.keep_score_step(state, ks, np.array([5, 99]), lam=0.5, req=[0])
