"""Pins for the oracle's budgeted top-k (CPU only).

The brute force maximises the kept set's score sum over every subset of the
right size (the arg-top of a sum in IntentKV §4), breaking ties toward the
lexicographically smallest index set, which is the lower-index rule.
"""
import itertools

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import select as osel

VALUES = [-2.0, -1.0, -0.0, 0.0, 0.5, 1.0, 3.0]     # dyadic: subset sums are exact


def brute_force(scores, k_total, n_sink, n_recent, alive):
    n = len(scores)
    forced = [j for j in range(n) if (j < n_sink or j >= n - n_recent) and alive[j]]
    alive_idx = [j for j in range(n) if alive[j]]
    if len(alive_idx) <= k_total:
        return alive_idx
    cand = [j for j in alive_idx if j not in forced]
    room = k_total - len(forced)
    best, best_key = None, None
    for sub in itertools.combinations(cand, room):
        total = sum(scores[j] for j in sub)
        key = (-total, tuple(sorted(sub)))
        if best_key is None or key < best_key:
            best, best_key = sub, key
    return sorted(forced + list(best))


@settings(max_examples=300, deadline=None)
@given(st.data())
def test_topk_equals_max_sum_brute_force(data):
    n = data.draw(st.integers(1, 10))
    scores = data.draw(st.lists(st.sampled_from(VALUES), min_size=n, max_size=n))
    alive = data.draw(st.lists(st.booleans(), min_size=n, max_size=n))
    n_sink = data.draw(st.integers(0, 3))
    n_recent = data.draw(st.integers(0, 3))
    k_total = data.draw(st.integers(0, n + 1))
    if k_total < n and n_sink + n_recent > k_total:
        with pytest.raises(osel.BudgetError):
            osel.select_topk(scores, k_total, n_sink, n_recent, alive)
        return
    kept, mask = osel.select_topk(scores, k_total, n_sink, n_recent, alive)
    assert kept.tolist() == brute_force(scores, k_total, n_sink, n_recent, alive)
    assert mask.tolist() == [j in set(kept.tolist()) for j in range(n)]


def test_negative_zero_ties_positive_zero():
    s = np.array([1.0, 0.0, -0.0, 0.0, -1.0])
    kept, _ = osel.select_topk(s, 2, 0, 0)
    assert kept.tolist() == [0, 1]
    s2 = np.array([1.0, -0.0, 0.0, -1.0])
    kept2, _ = osel.select_topk(s2, 2, 0, 0)
    assert kept2.tolist() == [0, 1]       # -0.0 at index 1 beats +0.0 at index 2


def test_invariants_on_random_units():
    r = np.random.default_rng(20)
    for _ in range(50):
        n = int(r.integers(50, 400))
        s = r.standard_normal(n).astype(np.float32)
        alive = r.random(n) > 0.1
        n_sink, n_recent = int(r.integers(0, 6)), int(r.integers(0, 20))
        k = int(r.integers(n_sink + n_recent, n))
        kept, mask = osel.select_topk(s, k, n_sink, n_recent, alive)
        forced = osel.forced_mask(n, n_sink, n_recent) & alive
        assert np.all(mask[forced])                       # sink and recent always kept
        assert not np.any(mask[~alive])                   # dead never revived
        assert len(kept) == min(k, int(alive.sum()))
        assert np.all(np.diff(kept) > 0)                  # chronological order
        rest = alive & ~forced
        if alive.sum() > k:
            assert s[mask & rest].min() >= s[~mask & rest].max()


@settings(max_examples=200, deadline=None)
@given(st.data())
def test_tiled_equals_untiled(data):
    n = data.draw(st.integers(1, 60))
    scores = data.draw(st.lists(st.sampled_from(VALUES), min_size=n, max_size=n))
    alive = data.draw(st.lists(st.booleans(), min_size=n, max_size=n))
    n_sink = data.draw(st.integers(0, 3))
    n_recent = data.draw(st.integers(0, 4))
    k_total = data.draw(st.integers(min(n_sink + n_recent, n), n + 2))
    tile = data.draw(st.integers(1, n + 3))
    a, ma = osel.select_topk(scores, k_total, n_sink, n_recent, alive)
    b, mb = osel.select_topk_tiled(scores, k_total, n_sink, n_recent, tile, alive)
    assert a.tolist() == b.tolist() and ma.tolist() == mb.tolist()


def test_budget_edge_cases():
    s = np.arange(10, dtype=float)
    kept, _ = osel.select_topk(s, 10, 3, 3)               # k >= N keeps all
    assert kept.tolist() == list(range(10))
    kept, _ = osel.select_topk(s, 12, 8, 8)               # overlapping F, k >= N
    assert kept.tolist() == list(range(10))
    kept, _ = osel.select_topk(s, 6, 3, 3)                # F fills the budget exactly
    assert kept.tolist() == [0, 1, 2, 7, 8, 9]
    with pytest.raises(osel.BudgetError):
        osel.select_topk(s, 5, 3, 3)
    kept, _ = osel.select_topk(s, 0, 0, 0)
    assert kept.tolist() == []
