"""Shared helpers for the GPU parity tests: device gating and the acceptance
rules that compare HIP outputs with the oracle.

Acceptance (stated once, used everywhere):
  * scores: per unit row, |gpu - oracle| <= 2e-3 * max(|oracle|, 1e-6 * max_j |oracle_j|),
    plus, for the signed block scores, the float32 error bound of the
    block scorer's arithmetic (block_score_tolerance): a dot product with
    cancellation is only accurate relative to the sum of its |terms|;
  * integer outputs (kept indices, masks, slot maps, page tables, counts):
    bit-exact, except when the oracle's float32 scores have a relative gap
    below 1e-5 between the last kept and the first dropped candidate; then
    the GPU set must still be a valid selection under the oracle's scores;
  * re-RoPEd K: element-wise |gpu - oracle| <= ULP_bf16(oracle element) +
    2^-20 * |pair| (|pair| = magnitude of the element's rotation pair: the
    float32 rotation with accurately reduced angles is within about 2^-21 of
    the pair's magnitude before its one rounding to bf16, so the two roundings
    can differ by one step of the element's own grid; the pair term only
    matters where a rotated element nearly cancels), and relative L2 per row
    <= 2e-3; unrotated K and all V bit-exact.
"""
import numpy as np
import pytest

from oracle import select as osel

SCORE_RTOL = 2e-3
TIE_RTOL = 1e-5
U32 = 2.0 ** -24          # unit roundoff of float32, round to nearest
U64 = 2.0 ** -53


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


def assert_scores_close(gpu, ora, what="scores", extra_tol=None):
    """``extra_tol`` (signed dot-product scores only): an additive bound of the
    same shape, from block_score_tolerance."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ora = np.asarray(ora, dtype=np.float64)
    assert gpu.shape == ora.shape, (gpu.shape, ora.shape)
    g2 = gpu.reshape(-1, gpu.shape[-1])
    o2 = ora.reshape(-1, ora.shape[-1])
    floor = 1e-6 * np.max(np.abs(o2), axis=1, keepdims=True)
    tol = SCORE_RTOL * np.maximum(np.abs(o2), floor)
    if extra_tol is not None:
        tol = tol + np.asarray(extra_tol, dtype=np.float64).reshape(o2.shape)
    bad = np.abs(g2 - o2) > tol
    if bad.any():
        r, c = np.argwhere(bad)[0]
        raise AssertionError("%s: %d elements out of tolerance; first at row %d col %d: gpu %r oracle %r"
                             % (what, int(bad.sum()), r, c, g2[r, c], o2[r, c]))


def gamma32(n_terms):
    """Relative bound, against the sum of |terms|, on the error of summing
    n_terms float32 numbers in any order with round-to-nearest:
    gamma_{n-1} = (n-1)u / (1 - (n-1)u) (Higham, Accuracy and Stability of
    Numerical Algorithms, the recursive-summation bound, which holds for every
    order and tree shape)."""
    k = max(int(n_terms) - 1, 0)
    return k * U32 / (1 - k * U32)


def gamma64(n_terms):
    k = max(int(n_terms) - 1, 0)
    return k * U64 / (1 - k * U64)


def qbar_error_bound(qbar_abs, q_abs_sum, n_terms):
    """Bound on |q-bar(GPU) - q-bar(exact)| per element: the library sums the
    n_terms query rows of a KV group in float64 and rounds once to float32.
    q_abs_sum = sum of |terms| per element."""
    return U32 * np.asarray(qbar_abs, np.float64) + (1 + U32) * gamma64(n_terms) * np.asarray(q_abs_sum, np.float64)


def block_score_tolerance(want, qbar_abs, mu, scale, qbar_err):
    """Additive float32 error bound of a block score s = scale * q-bar . mu.

    The library's arithmetic: q-bar in float32 (within ``qbar_err`` of the
    exact one); for D 128 it enters f16 matrix-core products as hi + lo parts
    of q-bar * 2^(14 - e) (|q-bar| < 2^e), whose residual is at most
    2^-22 |q-bar_d| plus 2^-38 max|q-bar| (the f16 subnormal floor); products
    of f16 values are exact in float32; the 2D partial products (D for the
    vector kernel) are summed in float32 in some order (gamma32(2D) of the
    sum of their |terms|); the result is scaled once by a rounded float32
    factor (2 roundings).  Arrays: qbar_abs and qbar_err [..., D], mu
    [..., n, D] (broadcasting as in matmul), want [..., n]."""
    mu_abs = np.abs(np.asarray(mu, np.float64))
    qa = np.asarray(qbar_abs, np.float64)
    qe = np.asarray(qbar_err, np.float64)
    D = qa.shape[-1]

    def dot(v):
        return (mu_abs @ v[..., :, None])[..., 0] * scale

    A = dot(qa + qe)                                   # sum of |terms| with the GPU's q-bar
    B = dot(qe)                                        # the q-bar error carried through
    floor = dot(np.broadcast_to(qa.max(axis=-1, keepdims=True), qa.shape)) * 2.0 ** -38
    rep = 2.0 ** -22
    return ((gamma32(2 * D) * (1 + 2.0 ** -10) + rep) * A + B + floor
            + 2 * U32 * (np.abs(np.asarray(want, np.float64)) + A))


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


def boundary_gap(scores32, k_total, n_sink, n_recent, alive=None):
    """The oracle's float32 relative gap between the last kept and the first
    dropped candidate of one unit (None when the selection does not depend on
    the scores: everything alive fits the budget, or nothing is left to fill)."""
    s = np.asarray(scores32, dtype=np.float64) + 0.0
    n = s.shape[0]
    alive_m = np.ones(n, bool) if alive is None else np.asarray(alive, bool)
    forced = osel.forced_mask(n, n_sink, n_recent) & alive_m
    cand = np.nonzero(alive_m & ~forced)[0]
    room = k_total - int(forced.sum())
    if not 0 < room < len(cand):
        return None
    top = np.partition(-s[cand], (room - 1, room))[[room - 1, room]]
    last_in, first_out = -top[0], -top[1]
    return (last_in - first_out) / max(abs(last_in), 1e-30)


class Conditioning:
    """How one configuration's selections compared with the oracle: units
    bit-exact, units accepted under the near-tie rule, units whose oracle
    boundary gap is below TIE_RTOL (near-tie) or exactly zero (exact tie),
    and units whose materialisation (gather, page table, redirect) was
    compared bit for bit.  report() is printed by the full-size tests."""

    def __init__(self, name):
        self.name = name
        self.units = self.exact = self.accepted = self.near = self.ties = self.materialised = 0

    def add(self, verdict, gap):
        self.units += 1
        self.exact += verdict == "exact"
        self.accepted += verdict == "near-tie"
        if gap is not None and gap < TIE_RTOL:
            self.near += 1
            self.ties += gap == 0.0

    def report(self):
        return ("conditioning %s: %d units compared, %d bit-exact, %d accepted as near-ties; oracle boundary "
                "gap < %g in %d units (exactly 0 in %d); materialisation compared bit for bit on %d units"
                % (self.name, self.units, self.exact, self.accepted, TIE_RTOL, self.near, self.ties,
                   self.materialised))


def _first_diff(a, b):
    m = min(len(a), len(b))
    for i in range(m):
        if a[i] != b[i]:
            return "position %d (gpu %d, oracle %d)" % (i, a[i], b[i])
    return "length"


def bf16_ulp(x):
    """ULP of the bf16 grid at each element's magnitude (0 at exact zeros)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    return np.where(a > 0, np.ldexp(1.0, np.frexp(a)[1] - 8), 0.0)


def pair_norm(x, style="half"):
    """Magnitude of each element's rotation pair: (m, m + D/2) for the
    rotate-half form, (2m, 2m + 1) for the interleaved form."""
    x = np.asarray(x, dtype=np.float64)
    if style == "half":
        h = x.shape[-1] // 2
        r = np.hypot(x[..., :h], x[..., h:])
        return np.concatenate([r, r], axis=-1)
    r = np.hypot(x[..., 0::2], x[..., 1::2])
    return np.repeat(r, 2, axis=-1)


ROPE_PAIR_RTOL = 2.0 ** -20


def rope_violations(gpu, ora, style="half"):
    """Boolean mask of the elements outside the per-element re-RoPE bar."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ora = np.asarray(ora, dtype=np.float64)
    tol = bf16_ulp(ora) + ROPE_PAIR_RTOL * pair_norm(ora, style)
    return np.abs(gpu - ora) > tol


def assert_rope_close(gpu, ora, what="rotated K", style="half"):
    gpu = np.asarray(gpu, dtype=np.float64)
    ora = np.asarray(ora, dtype=np.float64)
    bad = rope_violations(gpu, ora, style)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d elements beyond 1 ULP of the element + 2^-20 of its pair; first at %s: "
                             "gpu %r oracle %r" % (what, int(bad.sum()), i, gpu[i], ora[i]))
    num = np.linalg.norm((gpu - ora).reshape(-1, ora.shape[-1]), axis=1)
    den = np.maximum(np.linalg.norm(ora.reshape(-1, ora.shape[-1]), axis=1), 1e-30)
    assert np.all(num / den <= 2e-3), "%s: relative L2 %.3g > 2e-3" % (what, float((num / den).max()))
