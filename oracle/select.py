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
import numpy as np


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
