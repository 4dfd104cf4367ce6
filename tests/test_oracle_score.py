"""Pins for the oracle's scoring steps (CPU only).

Each test checks the oracle against something other than its own formula:
hand-computed closed forms, invariants the pages state, or a second
formulation that the pages say is equivalent.
"""
import math

import numpy as np
import pytest

from oracle import score


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- window scores

def test_two_key_closed_form_fixes_scale():
    # D = 4, q = (2,0,0,0), k0 = (1,0,0,0), k1 = 0: logits 2/sqrt(4) = 1 and 0
    q = np.zeros((1, 1, 1, 4)); q[0, 0, 0, 0] = 2.0
    k = np.zeros((1, 1, 2, 4)); k[0, 0, 0, 0] = 1.0
    a, lse = score.window_scores(q, k)
    e = math.e
    np.testing.assert_allclose(a[0, 0], [e / (1 + e), 1 / (1 + e)], rtol=0, atol=1e-15)
    assert abs(lse[0, 0, 0] - math.log(1 + e)) < 1e-15


def test_causal_window_rows_see_only_their_prefix():
    # N = 4, W = 2: row 0 sits at position 2, row 1 at position 3
    c = 3.0
    q = np.zeros((1, 1, 2, 2)); q[0, 0, :, 0] = 1.0
    k = np.zeros((1, 1, 4, 2)); k[0, 0, 3, 0] = c * math.sqrt(2)      # logit c for key 3
    a, _ = score.window_scores(q, k, causal=True)
    ec = math.exp(c)
    row0 = np.array([1, 1, 1, 0]) / 3.0
    row1 = np.array([1, 1, 1, ec]) / (3.0 + ec)
    np.testing.assert_allclose(a[0, 0], row0 + row1, atol=1e-15)
    a_nc, _ = score.window_scores(q, k, causal=False)
    np.testing.assert_allclose(a_nc[0, 0], 2 * row1, atol=1e-15)


def test_gqa_groups_are_consecutive_query_heads():
    # heads 0,1 look along e1, heads 2,3 along e2; KV head 0 has a key along e1
    # at j = 0, KV head 1 a key along e2 at j = 1
    N, D, c = 5, 2, 5.0
    q = np.zeros((1, 4, 1, D))
    q[0, 0:2, 0, 0] = 1.0
    q[0, 2:4, 0, 1] = 1.0
    k = np.zeros((1, 2, N, D))
    k[0, 0, 0, 0] = c
    k[0, 1, 1, 1] = c
    a, _ = score.window_scores(q, k)
    pk = math.exp(c / math.sqrt(D))
    peak, rest = pk / (pk + N - 1), 1 / (pk + N - 1)
    exp0 = np.full(N, 2 * rest); exp0[0] = 2 * peak
    exp1 = np.full(N, 2 * rest); exp1[1] = 2 * peak
    np.testing.assert_allclose(a[0, 0], exp0, atol=1e-15)
    np.testing.assert_allclose(a[0, 1], exp1, atol=1e-15)
    assert score.gqa_group(3, 32, 8) == 0 and score.gqa_group(4, 32, 8) == 1


def test_softmax_rows_sum_to_one_and_totals_equal_row_count():
    r = _rng(3)
    L, Hq, Hkv, W, N, D = 2, 8, 2, 5, 40, 16
    q = r.standard_normal((L, Hq, W, D)) * 2
    k = r.standard_normal((L, Hkv, N, D)) * 2
    a, lse = score.window_scores(q, k)
    np.testing.assert_allclose(a.sum(axis=-1), Hq // Hkv * W, rtol=1e-12)
    # each row's LSE normalises its own allowed logits
    for l in range(L):
        for h in range(Hq):
            g = score.gqa_group(h, Hq, Hkv)
            for t in range(W):
                s = k[l, g, :N - W + t + 1] @ q[l, h, t] / math.sqrt(D)
                assert abs(np.exp(s - lse[l, h, t]).sum() - 1.0) < 1e-12


def test_lse_recovery_equals_self_normalised_and_shifts_scale():
    r = _rng(4)
    q = r.standard_normal((1, 4, 3, 8))
    k = r.standard_normal((1, 2, 20, 8))
    a, lse = score.window_scores(q, k)
    a2, _ = score.window_scores(q, k, lse_in=lse)
    np.testing.assert_allclose(a2, a, rtol=1e-14)
    a3, _ = score.window_scores(q, k, lse_in=lse + 0.5)
    np.testing.assert_allclose(a3, a * math.exp(-0.5), rtol=1e-14)


def test_max_over_group_then_mean_over_rows():
    # two heads in one group, W = 2 rows, one-hot queries and keys with
    # logits 2, 1, 3 for the key each row prefers (0 elsewhere); head 0's two
    # rows prefer different keys, so max-then-mean and mean-then-max differ
    N, D = 3, 3
    q = np.zeros((1, 2, 2, D))
    q[0, 0, 0, 0] = 1.0           # head 0, row 0 -> key 0
    q[0, 0, 1, 2] = 1.0           # head 0, row 1 -> key 2
    q[0, 1, :, 1] = 1.0           # head 1, both rows -> key 1
    k = np.zeros((1, 1, N, D))
    for j, v in enumerate([2.0, 1.0, 3.0]):
        k[0, 0, j, j] = math.sqrt(D) * v
    a, _ = score.window_scores(q, k, causal=False, head_agg="max", row_agg="mean")
    e = math.e
    h0r0 = np.array([e ** 2, 1, 1]) / (e ** 2 + 2)
    h0r1 = np.array([1, 1, e ** 3]) / (e ** 3 + 2)
    h1 = np.array([1, e, 1]) / (e + 2)
    want = (np.maximum(h0r0, h1) + np.maximum(h0r1, h1)) / 2
    np.testing.assert_allclose(a[0, 0], want, atol=1e-15)
    assert not np.allclose(want, np.maximum((h0r0 + h0r1) / 2, h1))      # the order matters here
    s, _ = score.window_scores(q, k, causal=False, head_agg="sum", row_agg="mean")
    np.testing.assert_allclose(s[0, 0], (h0r0 + h0r1) / 2 + h1, atol=1e-15)


def test_planted_high_norm_keys_rank_first():
    # sanity only: keys scaled x8 that align with every query dominate
    r = _rng(5)
    N, D = 64, 16
    direction = r.standard_normal(D); direction /= np.linalg.norm(direction)
    q = (r.standard_normal((1, 4, 4, D)) + 3 * direction)
    k = r.standard_normal((1, 1, N, D))
    planted = np.array([7, 19, 33])
    k[0, 0, planted] = 8 * direction * math.sqrt(D) / 2
    a, _ = score.window_scores(q, k, causal=False)
    assert set(np.argsort(-a[0, 0])[:3].tolist()) == set(planted.tolist())


# ---------------------------------------------------------------- pooling

@pytest.mark.parametrize("pos", [0, 1, 5, 9])
def test_pool_impulse_response(pos):
    N, ks = 10, 7
    a = np.zeros(N); a[pos] = 1.0
    cover = (np.abs(np.arange(N) - pos) <= 3)
    np.testing.assert_allclose(score.pool1d(a, "avg", ks), cover / 7.0, atol=0)
    np.testing.assert_array_equal(score.pool1d(a, "max", ks), cover.astype(float))


def test_pool_avg_total_is_coverage_weighted():
    r = _rng(6)
    N, ks = 50, 7
    a = r.random(N)
    j = np.arange(N)
    cover = np.minimum(j, 3) + np.minimum(N - 1 - j, 3) + 1
    assert abs(score.pool1d(a, "avg", ks).sum() - (a * cover).sum() / ks) < 1e-12
    m = score.pool1d(a, "max", ks)
    assert np.all(m >= a) and m.max() == a.max()


# ---------------------------------------------------------------- query memory

def test_memory_two_turn_closed_form():
    m0 = np.zeros((1, 1, 2))
    t1 = np.array([[[[2.0, 4.0], [4.0, 4.0]]]])        # mean (3, 4)
    m1 = score.memory_update(m0, t1)
    np.testing.assert_allclose(m1[0, 0], [0.6, 0.8], atol=1e-15)
    t2 = np.array([[[[0.0, 0.0], [2.0, 0.0]]]])        # mean (1, 0), sum (2, 0)
    m2 = score.memory_update(m1, t2, decay=0.9)
    np.testing.assert_allclose(m2[0, 0], [1.54 / 1.7, 0.72 / 1.7], atol=1e-15)


def test_memory_unit_norm_fixed_point_and_zero():
    r = _rng(7)
    L, Hq, W, D = 2, 3, 4, 8
    m = np.zeros((L, Hq, D))
    for _ in range(8):
        m = score.memory_update(m, r.standard_normal((L, Hq, W, D)))
        np.testing.assert_allclose(np.linalg.norm(m, axis=-1), 1.0, atol=1e-14)
    e = r.standard_normal((L, Hq, D))
    turn = np.repeat(e[:, :, None, :], W, axis=2)
    u = e / np.linalg.norm(e, axis=-1, keepdims=True)
    np.testing.assert_allclose(score.memory_update(u, turn), u, atol=1e-14)
    z = score.memory_update(np.zeros((1, 1, 4)), np.zeros((1, 1, 2, 4)))
    assert np.all(z == 0)


def test_unnormalised_memory_norm_grows_linearly_without_decay():
    # negative control for the unit-norm projection: with decay 1 and no
    # renormalisation the norm after t identical turns is t * |e|
    e = np.array([3.0, 4.0])
    m = np.zeros(2)
    for t in range(1, 6):
        m = 1.0 * m + e
        assert abs(np.linalg.norm(m) - 5.0 * t) < 1e-12


def _memory_inputs(seed, L=2, Hq=4, Hkv=2, ps=4, n_pages=6, D=8, extra_pages=2):
    r = _rng(seed)
    N = ps * n_pages
    m = score.memory_update(np.zeros((L, Hq, D)), r.standard_normal((L, Hq, 3, D)))
    P = n_pages + extra_pages
    pool = r.standard_normal((L, P, ps, Hkv, D))
    page_table = r.permutation(P)[:n_pages]
    return m, pool, page_table, N


def test_memory_scores_equal_single_row_window_scores():
    m, pool, pt, N = _memory_inputs(8)
    L, Hq, D = m.shape
    Hkv, ps = pool.shape[3], pool.shape[2]
    rule = score.memory_scores(m, pool, pt, ps, N)
    j = np.arange(N)
    klog = np.stack([np.transpose(pool[l][pt[j // ps], j % ps], (1, 0, 2)) for l in range(L)])
    a, _ = score.window_scores(m[:, :, None, :], klog)        # W = 1 sees every key
    np.testing.assert_allclose(rule, a.sum(axis=(0, 1)), rtol=1e-13)
    per_unit = score.memory_scores(m, pool, pt, ps, N, reduce="per_unit")
    np.testing.assert_allclose(per_unit, a, rtol=1e-13)
    assert abs(rule.sum() - L * Hq) < 1e-12


def test_memory_scores_history_excludes_forced_and_dead():
    m, pool, pt, N = _memory_inputs(9)
    L, Hq, D = m.shape
    ps = pool.shape[2]
    dead = 10_000
    slot_map = (pt[np.arange(N) // ps] * ps + np.arange(N) % ps).astype(np.int64)
    slot_map[[5, 6, 11]] = dead
    n_sink, n_recent = 2, 3
    rule = score.memory_scores(m, pool, pt, ps, N, slot_map=slot_map, dead_slot=dead,
                               n_sink=n_sink, n_recent=n_recent)
    hist = np.ones(N, bool)
    hist[:n_sink] = False; hist[N - n_recent:] = False; hist[[5, 6, 11]] = False
    assert np.all(rule[~hist] == 0)
    assert abs(rule.sum() - L * Hq) < 1e-12
    # same as scoring only the history keys with a single-row window
    j = np.nonzero(hist)[0]
    klog = np.stack([np.transpose(pool[l][pt[j // ps], j % ps], (1, 0, 2)) for l in range(L)])
    a, _ = score.window_scores(m[:, :, None, :], klog)
    np.testing.assert_allclose(rule[hist], a.sum(axis=(0, 1)), rtol=1e-13)


def test_zero_initialised_residual_is_rule_exactly():
    r = _rng(10)
    n, fdim, hid = 30, 13, 16
    rule = r.random(n)
    feats = r.standard_normal((n, fdim))
    s = score.residual_score(rule, feats, r.standard_normal((hid, fdim)), r.standard_normal(hid),
                             np.zeros((1, hid)), np.zeros(1), alpha=1.0)
    np.testing.assert_array_equal(s, rule)
    s2 = score.residual_score(rule, feats, r.standard_normal((hid, fdim)), r.standard_normal(hid),
                              r.standard_normal((1, hid)), np.zeros(1), alpha=1.0)
    assert np.any(s2 != rule)


# ---------------------------------------------------------------- block scores

def test_block_scores_equal_per_query_brute_force():
    r = _rng(11)
    S, L, Hq, Hkv, Wq, D, NB = 2, 2, 4, 2, 3, 4, 5
    q = r.standard_normal((S, L, Hq, Wq, D))
    mu = r.standard_normal((L, Hkv, NB, D))
    got = score.block_scores(score.query_reduce(q, Hkv), mu)
    want = np.zeros((S, L, Hkv, NB))
    for s in range(S):
        for l in range(L):
            for h in range(Hq):
                g = h // (Hq // Hkv)
                for t in range(Wq):
                    for b in range(NB):
                        want[s, l, g, b] += float(np.dot(q[s, l, h, t], mu[l, g, b])) / math.sqrt(D)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_block_score_of_mean_k_is_mean_of_token_scores():
    # with mu built as the mean of a block's raw keys, the block score is the
    # mean over the block's tokens of q-bar . k / sqrt(D)
    r = _rng(12)
    D, bt, NB = 8, 32, 4
    raw = r.standard_normal((NB, bt, D))
    mu = raw.mean(axis=1)
    q = r.standard_normal((1, 1, 2, 5, D))
    qbar = score.query_reduce(q, 1)
    got = score.block_scores(qbar, mu[None, None])[0, 0, 0]
    want = (raw @ qbar[0, 0, 0]).mean(axis=1) / math.sqrt(D)
    np.testing.assert_allclose(got, want, rtol=1e-12)


def test_block_score_hand_example():
    q = np.zeros((1, 1, 2, 2, 4))
    q[0, 0, 0, 0] = [1, 0, 0, 0]; q[0, 0, 0, 1] = [1, 1, 0, 0]
    q[0, 0, 1, 0] = [0, 0, 2, 0]; q[0, 0, 1, 1] = [0, 0, 0, -1]
    mu = np.zeros((1, 1, 2, 4)); mu[0, 0, 0] = [1, 1, 1, 1]; mu[0, 0, 1] = [0, 0, 0, 4]
    got = score.block_scores(score.query_reduce(q, 1), mu)[0, 0, 0]
    # q-bar = (2, 1, 2, -1); / sqrt(4) = 2
    np.testing.assert_allclose(got, [4.0 / 2, -4.0 / 2], atol=0)


# ---------------------------------------------------------------- Mean-K index

def test_mean_k_hand_example_two_blocks():
    # bt = 4, D = 2: block 0 rows (1,2),(3,4),(5,6),(7,8) -> (4,5);
    # block 1 rows (0,-1),(0,-1),(2,1),(2,-3) -> (1,-1); a trailing partial row is ignored
    raw = np.array([[1, 2], [3, 4], [5, 6], [7, 8],
                    [0, -1], [0, -1], [2, 1], [2, -3],
                    [100, 100]], dtype=np.float64)
    mu = score.mean_k_index(raw, bt=4)
    assert mu.shape == (2, 2)
    np.testing.assert_array_equal(mu, [[4.0, 5.0], [1.0, -1.0]])


def test_mean_k_rounds_once_to_float16_nearest_even():
    # half spacing at 1.0 is 2^-10.  Means exactly between two halves go to the
    # even one; the fp16 value of 0.1 is 0x2E66 = 0.0999755859375.
    u = 2.0 ** -10
    raw = np.array([[1.0], [1.0 + u],              # mean 1 + u/2 -> 1.0 (even)
                    [1.0 + u], [1.0 + 2 * u],      # mean 1 + 3u/2 -> 1 + 2u (even)
                    [0.1], [0.1],                  # constant block
                    [70000.0], [70000.0]])         # beyond the half range -> inf
    mu = score.mean_k_index(raw, bt=2)[:, 0]
    assert mu[0] == 1.0 and mu[1] == 1.0 + 2 * u
    assert mu[2] == 0.0999755859375
    assert np.isinf(mu[3]) and mu[3] > 0
    # below the halfway point of the subnormal spacing 2^-24 the mean flushes to zero
    tiny = score.mean_k_index(np.array([[2.0 ** -26], [2.0 ** -26]]), bt=2)
    assert tiny[0, 0] == 0.0


def test_mean_k_block_score_equals_mean_of_token_scores():
    # linearity: scoring the mean key of a block is scoring each of its tokens
    # and averaging; raw values on a 2^-4 grid keep every mean exact in fp16
    r = _rng(21)
    L, Hkv, NB, bt, D = 1, 2, 3, 32, 8
    raw = r.integers(-64, 64, size=(L, Hkv, NB * bt, D)) / 16.0
    mu = score.mean_k_index(raw, bt=bt)
    np.testing.assert_array_equal(mu, raw.reshape(L, Hkv, NB, bt, D).mean(axis=3))
    qbar = r.standard_normal((1, L, Hkv, D))
    got = score.block_scores(qbar, mu)
    tok = np.einsum("slgd,lgnd->slgn", qbar, raw).reshape(1, L, Hkv, NB, bt).mean(axis=-1) / math.sqrt(D)
    np.testing.assert_allclose(got, tok, rtol=1e-12, atol=1e-12)
