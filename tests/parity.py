"""Shared helpers for the GPU parity tests: device gating and the acceptance
rules that compare HIP outputs with the oracle.

Acceptance (stated once, used everywhere):
  * scores: per unit row, |gpu - oracle| <= 2e-3 * max(|oracle|, 1e-6 * max_j |oracle_j|),
    plus 1e-5 * sum_d |q_d mu_d| / sqrt(D) for the signed block scores (a
    dot product with cancellation is only accurate relative to its terms);
  * integer outputs (kept indices, masks, slot maps, page tables, counts):
    bit-exact, except when the oracle's float32 scores have a relative gap
    below 1e-5 between the last kept and the first dropped candidate; then
    the GPU set must still be a valid selection under the oracle's scores;
  * re-RoPEd K: within 1 bf16 ULP of the oracle element-wise (ULP of the
    element's rotate-half pair magnitude) and relative L2 per row <= 2e-3;
    unrotated K and all V bit-exact.
"""
import numpy as np
import pytest

from oracle import select as osel

SCORE_RTOL = 2e-3
MAG_RTOL = 1e-5
TIE_RTOL = 1e-5


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from selection_score_amd import _abi
    _abi.load()            # raises if the library is missing: no silent fallback
    return torch.device("cuda:0")


def f64(t):
    """torch tensor (any dtype, any device) -> float64 numpy, exactly."""
    return t.detach().to("cpu").to(dtypes_f32(t)).numpy().astype(np.float64)


def dtypes_f32(t):
    import torch
    return torch.float64 if t.dtype == torch.float64 else torch.float32


def assert_scores_close(gpu, ora, what="scores", mag=None):
    """``mag`` (signed dot-product scores only): the oracle's sum of |terms| of
    each score; a float32 sum with cancellation can only be accurate relative
    to it, so MAG_RTOL * mag is added to the bound."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ora = np.asarray(ora, dtype=np.float64)
    assert gpu.shape == ora.shape, (gpu.shape, ora.shape)
    g2 = gpu.reshape(-1, gpu.shape[-1])
    o2 = ora.reshape(-1, ora.shape[-1])
    floor = 1e-6 * np.max(np.abs(o2), axis=1, keepdims=True)
    tol = SCORE_RTOL * np.maximum(np.abs(o2), floor)
    if mag is not None:
        tol = tol + MAG_RTOL * np.asarray(mag, dtype=np.float64).reshape(o2.shape)
    bad = np.abs(g2 - o2) > tol
    if bad.any():
        r, c = np.argwhere(bad)[0]
        raise AssertionError("%s: %d elements out of tolerance; first at row %d col %d: gpu %r oracle %r"
                             % (what, int(bad.sum()), r, c, g2[r, c], o2[r, c]))


def check_selection(gpu_kept, scores32, k_total, n_sink, n_recent, alive=None, what="selection"):
    """Compare one unit's GPU kept list with the oracle's selection on the
    oracle's float32 scores, with the near-tie rule.  Returns "exact" or
    "near-tie"."""
    s = np.asarray(scores32, dtype=np.float64) + 0.0
    n = s.shape[0]
    gpu_kept = np.asarray(gpu_kept, dtype=np.int64)
    gpu_kept = gpu_kept[gpu_kept >= 0]
    ora_kept, _ = osel.select_topk(s, k_total, n_sink, n_recent, alive)
    if gpu_kept.shape == ora_kept.shape and np.array_equal(gpu_kept, ora_kept):
        return "exact"
    alive_m = np.ones(n, bool) if alive is None else np.asarray(alive, bool)
    forced = osel.forced_mask(n, n_sink, n_recent) & alive_m
    cand = np.nonzero(alive_m & ~forced)[0]
    room = k_total - int(forced.sum())
    order = cand[np.lexsort((cand, -s[cand]))]
    assert 0 < room < len(order), "%s differs where the selection is not score-dependent" % what
    last_in, first_out = s[order[room - 1]], s[order[room]]
    gap = (last_in - first_out) / max(abs(last_in), 1e-30)
    assert gap < TIE_RTOL, ("%s differs with a boundary gap of %.3g (>= %g): gpu %d kept, oracle %d; "
                            "first difference at %s" % (what, gap, TIE_RTOL, len(gpu_kept),
                                                        len(ora_kept), _first_diff(gpu_kept, ora_kept)))
    gk = set(gpu_kept.tolist())
    assert len(gpu_kept) == len(ora_kept) and np.all(np.diff(gpu_kept) > 0)
    assert set(np.nonzero(forced)[0].tolist()) <= gk
    assert all(alive_m[j] for j in gk)
    sel = np.array([j for j in cand if j in gk], dtype=np.int64)
    uns = np.array([j for j in cand if j not in gk], dtype=np.int64)
    assert s[sel].min() >= s[uns].max() - TIE_RTOL * abs(last_in), "%s: invalid near-tie set" % what
    return "near-tie"


def _first_diff(a, b):
    m = min(len(a), len(b))
    for i in range(m):
        if a[i] != b[i]:
            return "position %d (gpu %d, oracle %d)" % (i, a[i], b[i])
    return "length"


def bf16_pair_ulp(x):
    """ULP of bf16 at each rotate-half pair's magnitude (per element)."""
    h = x.shape[-1] // 2
    r = np.sqrt(x[..., :h] ** 2 + x[..., h:] ** 2)
    r = np.concatenate([r, r], axis=-1)
    return np.ldexp(1.0, np.frexp(r)[1] - 8)


def assert_rope_close(gpu, ora, what="rotated K"):
    gpu = np.asarray(gpu, dtype=np.float64)
    ora = np.asarray(ora, dtype=np.float64)
    err = np.abs(gpu - ora)
    ulp = bf16_pair_ulp(ora)
    bad = err > ulp
    assert not bad.any(), "%s: %d elements beyond 1 ULP; worst %.3g ULP" % (
        what, int(bad.sum()), float((err / ulp).max()))
    num = np.linalg.norm((gpu - ora).reshape(-1, ora.shape[-1]), axis=1)
    den = np.maximum(np.linalg.norm(ora.reshape(-1, ora.shape[-1]), axis=1), 1e-30)
    assert np.all(num / den <= 2e-3), "%s: relative L2 %.3g > 2e-3" % (what, float((num / den).max()))
