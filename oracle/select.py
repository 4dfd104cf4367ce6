"""Budgeted top-k with a forced set.  Test infrastructure only.

IntentKV §4 (top-k selection): the kept set is the forced set F united with
the C* highest-scoring remaining positions, filling whatever budget F leaves.
KVMem (query-conditioned retrieval): sink and recent blocks are always kept,
the rest of the budget is filled by score, and the kept set is restored to
chronological order.  ActKV §3.3: entry eviction turns scores and a budget
into a Boolean keep mask.  IntentKV §3: a position already redirected to the
dead slot cannot be revived, so dead positions are never candidates.

Readings where the pages are silent: the budget counts the forced set; when
scores tie the lower position wins; -0.0 and +0.0 are the same score; when
no more positions are alive than the budget allows, all of them are kept.
"""
import math

import numpy as np

from . import numerics


class BudgetError(ValueError):
    """n_sink + n_recent exceeds the budget while the budget is below N."""


def forced_mask(n, n_sink, n_recent):
    j = np.arange(n)
    return (j < n_sink) | (j >= n - n_recent)


def select_topk(scores, k_total, n_sink, n_recent, alive=None):
    """Kept positions (ascending int64) and the keep mask (bool) of one unit.

    scores: [N] (compared as given; pass float32-rounded values to mirror a
    float32 pipeline).  alive: optional [N] bool (False = dead).
    """
    s = np.asarray(scores, dtype=np.float64) + 0.0      # -0.0 + 0.0 == +0.0
    n = s.shape[0]
    if k_total < n and n_sink + n_recent > k_total:
        raise BudgetError("forced set larger than the budget")
    alive = np.ones(n, dtype=bool) if alive is None else np.asarray(alive, dtype=bool)
    keep = np.zeros(n, dtype=bool)
    if alive.sum() <= k_total:
        keep[:] = alive
    else:
        f = forced_mask(n, n_sink, n_recent) & alive
        keep |= f
        cand = np.nonzero(alive & ~f)[0]
        room = k_total - int(f.sum())
        order = np.lexsort((cand, -s[cand]))            # score desc, index asc
        keep[cand[order[:room]]] = True
    return np.nonzero(keep)[0].astype(np.int64), keep


def select_topk_tiled(scores, k_total, n_sink, n_recent, tile, alive=None):
    """Streaming form: candidates merged tile by tile into a running top-k'.

    Defined to equal ``select_topk`` (KVMem scores its index in bounded tiles);
    kept here so the equality can be checked for every tile size.
    """
    s = np.asarray(scores, dtype=np.float64) + 0.0
    n = s.shape[0]
    if k_total < n and n_sink + n_recent > k_total:
        raise BudgetError("forced set larger than the budget")
    alive = np.ones(n, dtype=bool) if alive is None else np.asarray(alive, dtype=bool)
    if alive.sum() <= k_total:
        return np.nonzero(alive)[0].astype(np.int64), alive.copy()
    f = forced_mask(n, n_sink, n_recent) & alive
    room = k_total - int(f.sum())
    run_idx = np.zeros(0, dtype=np.int64)
    for b in range(0, n, tile):
        j = np.arange(b, min(n, b + tile))
        j = j[alive[j] & ~f[j]]
        pool = np.concatenate([run_idx, j])
        order = np.lexsort((pool, -s[pool]))
        run_idx = pool[order[:room]]
    keep = f.copy()
    keep[run_idx] = True
    return np.nonzero(keep)[0].astype(np.int64), keep


def action_scores(state, r, n_len):
    """Action-region attention score of each entry of request r.

    ActKV §5.2 scores an entry by the attention it received over the action
    region; the scorer keeps one running mean per (layer, KV head, position),
    and an entry is a position of the request across all layers and heads
    (the keep mask and the compaction act on positions).  Reading: the
    entry's score is the sum over layers and KV heads of those means, taken
    exactly and rounded once to float32 (the precision in which the entries
    are then ranked).  state: [L][R][Hkv][n_cap].  Returns [n_len] float64
    values representable in float32.
    """
    st = np.asarray(state, dtype=np.float64)[:, r, :, :n_len]
    L, Hkv = st.shape[0], st.shape[1]
    out = np.empty(n_len)
    for j in range(n_len):
        out[j] = math.fsum(st[:, :, j].reshape(L * Hkv).tolist())
    return numerics.round_to_f32(out)


def top_p_hits(scores, top_p=0.9):
    """Top-p hit mask: the shortest prefix of the entries, ordered by score
    descending (lower index first on ties), whose cumulative score reaches
    top_p times the total (ActKV §5.2: an entry is hit when its score falls in
    the top-p set; §5.1 uses the same set for the action access vector).

    Cumulative sums are taken in float64 in that order, and the total is the
    last of them.  A zero total (or top_p * total == 0) gives no hits.
    scores: [n] non-negative.  Returns [n] bool.
    """
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    hit = np.zeros(n, dtype=bool)
    if n == 0:
        return hit
    order = np.lexsort((np.arange(n), -s))
    cum = np.cumsum(s[order])
    target = top_p * cum[-1]
    if not target > 0.0:
        return hit
    m = int(np.searchsorted(cum, target, side="left")) + 1    # first prefix with cum >= target
    hit[order[:min(m, n)]] = True
    return hit


def lrfu_keep_score(ks, scores, hits, lam):
    """Attention-aware LRFU keep-score update of ActKV §5.2.

    The page's update equation is lost; the reading used is
        KS_t(i) = lam * KS_{t-1}(i) + hit_t(i) * AttnScore_t(i),
    which has the two limits the page describes: lam = 0 keeps only the
    latest step (recency), lam = 1 accumulates every hit without decay
    (frequency).  Parity unpinned for 0 < lam < 1: the page fixes those two
    limits and, in between, only the behaviour (a quiet intermittent entry
    with high attention survives, a stale continuous entry is overtaken).
    """
    ks = np.asarray(ks, dtype=np.float64)
    return lam * ks + np.where(hits, np.asarray(scores, dtype=np.float64), 0.0)


def keep_score_step(state, ks, n_len, *, lam, top_p=0.9, req=None):
    """One compression step of the ActKV policy for the requests in ``req``.

    Per request r: AttnScore = action_scores (entries j < n_len[r]), hits =
    top_p_hits, KS <- lrfu_keep_score.  A request holds at most n_cap
    entries, so an n_len of a listed request outside [0, n_cap] is an error.
    Returns (ks [R][n_cap] float64,
    hit [R][n_cap] bool, attn [R][n_cap] float64); entries j >= n_len[r]
    keep their KS and report no hit and score 0; requests not in ``req`` are
    unchanged with no hits and score 0.
    """
    ks_new = np.array(ks, dtype=np.float64)
    R, n_cap = ks_new.shape
    hit = np.zeros((R, n_cap), dtype=bool)
    attn = np.zeros((R, n_cap))
    req = np.arange(R) if req is None else np.asarray(req, dtype=np.int64)
    for r in req:
        r = int(r)
        n = int(n_len[r])
        if not 0 <= n <= n_cap:
            raise ValueError("n_len[%d] = %d lies outside [0, %d]" % (r, n, n_cap))
        a = action_scores(state, r, n)
        h = top_p_hits(a, top_p)
        ks_new[r, :n] = lrfu_keep_score(ks_new[r, :n], a, h, lam)
        hit[r, :n] = h
        attn[r, :n] = a
    return ks_new, hit, attn
