"""Scoring steps of the selection path.  Test infrastructure only.

All arithmetic in float64.  Callers round to float32 with
``numerics.round_to_f32`` when comparing with the GPU's float32 outputs.

Layouts (row-major, last index fastest):
  window queries   q      [L][Hq][W][D]     (post-RoPE, the last W positions)
  contiguous keys  k      [L][Hkv][N][D]
  query memory     M      [L][Hq][D]
  block queries    q      [S][L][Hq][Wq][D] (pre-RoPE)
  Mean-K index     mu     [L][Hkv][NB][D]
  raw keys         raw_k  [..., NB*bt, D]   (pre-RoPE, bt-token blocks)
  decode queries   q      [L][Ra][Hq][D]    (post-RoPE, one token per request)
  paged KV pool    k_pool [L][P][BS][Hkv][D]
  running means    state  [L][R][Hkv][n_cap]
"""
import numpy as np

from . import numerics


def gqa_group(h, n_q_heads, n_kv_heads):
    """KV head serving query head ``h`` under grouped-query attention.

    ActKV §7.1 (Algorithm 3 reduces over the query heads of one KV head's
    group) and IntentKV §4 minimum check 1 (KV heads expanded to the query
    heads): consecutive blocks of Hq/Hkv query heads share one KV head.
    """
    return h // (n_q_heads // n_kv_heads)


def _logsumexp(s, allowed):
    """log sum_j exp(s_j) over allowed j, max-shifted (ActKV §7.1, the LSE)."""
    neg = np.where(allowed, s, -np.inf)
    m = np.max(neg, axis=-1, keepdims=True)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    tot = np.sum(np.where(allowed, np.exp(neg - m_safe), 0.0), axis=-1, keepdims=True)
    return (m_safe + np.log(tot))[..., 0]


def _reduce(x, how, axis):
    if how == "sum":
        return np.sum(x, axis=axis)
    if how == "mean":
        return np.mean(x, axis=axis)
    if how == "max":
        return np.max(x, axis=axis)
    raise ValueError(how)


def window_scores(q, k, *, scale=None, causal=True, lse_in=None,
                  head_agg="sum", row_agg="sum"):
    """Token scores of every cached key against a query window.

    ActKV §2: the attention score of a cached key is its softmax weight,
    softmax(q . k / sqrt(D)) over the keys the query can see.  ActKV §7.1: the
    same probabilities are recovered as exp(s - LSE) from a log-sum-exp that
    the attention pass already produced; ``lse_in`` ([L][Hq][W]) takes that
    form, otherwise the LSE is computed here over the allowed keys.

    Window row t sits at position N - W + t and (if ``causal``) sees keys
    j <= N - W + t.  Per unit (layer l, KV head g) the probabilities of the
    group's query heads are combined with ``head_agg`` and then the window
    rows with ``row_agg`` (sum/sum is the SnapKV/H2O accumulation named in
    ActKV §2; max over the GQA group then mean over query tokens is
    Algorithm 3's form).

    Returns (scores [L][Hkv][N], lse [L][Hq][W]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    L, Hq, W, D = q.shape
    Lk, Hkv, N, Dk = k.shape
    assert Lk == L and Dk == D and Hq % Hkv == 0 and W <= N
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    pos = N - W + np.arange(W)
    if causal:
        allowed = np.arange(N)[None, :] <= pos[:, None]          # [W][N]
    else:
        allowed = np.ones((W, N), dtype=bool)
    scores = np.zeros((L, Hkv, N))
    lse_all = np.zeros((L, Hq, W))
    for l in range(L):
        for g in range(Hkv):
            heads = [h for h in range(Hq) if gqa_group(h, Hq, Hkv) == g]
            s = np.stack([q[l, h] @ k[l, g].T for h in heads]) * scale   # [G][W][N]
            if lse_in is None:
                lse = _logsumexp(s, allowed[None])                      # [G][W]
            else:
                lse = np.asarray(lse_in, dtype=np.float64)[l, heads]
            p = np.where(allowed[None], np.exp(s - lse[..., None]), 0.0)
            scores[l, g] = _reduce(_reduce(p, head_agg, 0), row_agg, 0)
            lse_all[l, heads] = lse
    assert len(heads) == G
    return scores, lse_all


def pool1d(a, kind, ksize):
    """Centred 1-D pooling along the last axis, stride 1, same length.

    ``kind`` "avg": (1/ksize) * sum of the in-range window (out-of-range terms
    count as zero); "max": maximum over the in-range window.  ``ksize`` odd.
    """
    a = np.asarray(a, dtype=np.float64)
    assert ksize % 2 == 1
    if kind == "none" or ksize == 1:
        return a.copy()
    r = ksize // 2
    N = a.shape[-1]
    idx = np.arange(N)
    if kind == "avg":
        out = np.zeros_like(a)
        for off in range(-r, r + 1):
            src = idx + off
            ok = (src >= 0) & (src < N)
            out[..., ok] += a[..., src[ok]]
        return out / ksize
    if kind == "max":
        out = np.full_like(a, -np.inf)
        for off in range(-r, r + 1):
            src = idx + off
            ok = (src >= 0) & (src < N)
            out[..., ok] = np.maximum(out[..., ok], a[..., src[ok]])
        return out
    raise ValueError(kind)


def memory_update(m_prev, q_turn, decay=0.9):
    """One turn of the session query memory.

    IntentKV §4 (memory recurrence) and §7 (unit-norm projection):
    M_t = normalise(decay * M_{t-1} + Enc(q_t)), normalised to unit L2 norm
    along the head dimension.  Enc is read as the mean of the turn's query
    rows per (layer, query head); a zero vector stays zero.

    m_prev: [L][Hq][D]; q_turn: [L][Hq][W][D].  Returns [L][Hq][D].
    """
    m_prev = np.asarray(m_prev, dtype=np.float64)
    e = np.mean(np.asarray(q_turn, dtype=np.float64), axis=2)
    m = decay * m_prev + e
    n = np.sqrt(np.sum(m * m, axis=-1, keepdims=True))
    return np.where(n > 0, m / np.where(n > 0, n, 1.0), 0.0)


def history_mask(n, n_sink, n_recent, slot_map=None, dead_slot=None):
    """Positions that are neither forced (sink, recent) nor dead."""
    j = np.arange(n)
    forced = (j < n_sink) | (j >= n - n_recent)
    alive = np.ones(n, dtype=bool) if slot_map is None else \
        (np.asarray(slot_map, dtype=np.int64) != dead_slot)
    return alive & ~forced


def memory_scores(m, k_pool, page_table, page_size, n, *, slot_map=None,
                  dead_slot=None, n_sink=0, n_recent=0, scale=None,
                  reduce="global"):
    """Memory-attention rule score over a paged KV pool.

    IntentKV §4 (rule score): for every layer l and query head h,
    a[l,h,j] = softmax over the history set H of M[l,h] . K[l,g(h),j] / sqrt(D),
    and rule_j = sum over (l, h) of a[l,h,j].  H excludes the forced set
    (sink and recent) and positions already redirected to the dead slot
    (IntentKV §3: eviction is one-way).  Positions outside H score 0.

    m: [L][Hq][D]; k_pool: [L][P][page_size][Hkv][D]; page_table: logical page
    -> physical page.  ``reduce`` "global" returns [N]; "per_unit" returns
    [L][Hkv][N] (sum over the group's heads only).
    """
    m = np.asarray(m, dtype=np.float64)
    L, Hq, D = m.shape
    Hkv = k_pool.shape[3]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    H = history_mask(n, n_sink, n_recent, slot_map, dead_slot)
    pt = np.asarray(page_table, dtype=np.int64)
    j = np.arange(n)
    phys_page = pt[j // page_size]
    in_page = j % page_size
    out = np.zeros(n) if reduce == "global" else np.zeros((L, Hkv, n))
    # logical position j lives in physical slot page_table[j // ps] * ps + j % ps
    slot = phys_page * page_size + in_page
    for l in range(L):
        flat = np.asarray(k_pool[l], dtype=np.float64).reshape(-1, Hkv, D)   # [slots][Hkv][D]
        for h in range(Hq):
            g = gqa_group(h, Hq, Hkv)
            s = ((flat[:, g, :] @ m[l, h]) * scale)[slot]      # logits in logical order
            lse = _logsumexp(s, H)
            p = np.where(H, np.exp(s - lse), 0.0)
            if reduce == "global":
                out += p
            else:
                out[l, g] += p
    return out


def query_reduce(q, n_kv_heads):
    """q-bar[s,l,g] = sum over window tokens t and heads h of group g of q.

    KVMem (query-conditioned retrieval) scores blocks in the model's own
    attention space with pre-RoPE queries; summing the queries first is the
    linearity of the dot product.  q: [S][L][Hq][Wq][D] -> [S][L][Hkv][D].
    """
    q = np.asarray(q, dtype=np.float64)
    S, L, Hq, Wq, D = q.shape
    out = np.zeros((S, L, n_kv_heads, D))
    for h in range(Hq):
        out[:, :, gqa_group(h, Hq, n_kv_heads)] += q[:, :, h].sum(axis=2)
    return out


def block_scores(qbar, mu, scale=None):
    """Block score s[s,l,g,b] = q-bar[s,l,g] . mu[l,g,b] / sqrt(D).

    KVMem (query-conditioned retrieval): one RoPE-stripped Mean-K vector per
    (layer, KV head, 32-token block), scored by a dot product with the query.
    qbar: [S][L][Hkv][D]; mu: [L][Hkv][NB][D].  Returns [S][L][Hkv][NB].
    """
    qbar = np.asarray(qbar, dtype=np.float64)
    mu = np.asarray(mu, dtype=np.float64)
    D = qbar.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    return np.einsum("slgd,lgbd->slgb", qbar, mu) * scale


def mean_k_index(raw_k, bt=32):
    """Mean-K index: mu[..., b, :] = (1/bt) * sum of the bt raw key rows of
    block b, rounded once (round-to-nearest-even) to float16.

    KVMem (query-conditioned retrieval paragraph): every (layer, KV head)
    keeps one RoPE-stripped mean key per 32-token block, stored in HBM as an
    fp16 index that grows as blocks fill.  raw_k: [..., N, D] with N >= 0;
    only the floor(N / bt) complete blocks are indexed.  Returns
    [..., N // bt, D] as float64 values representable in float16.
    """
    raw = np.asarray(raw_k, dtype=np.float64)
    *lead, n, d = raw.shape
    nb = n // bt
    blocks = raw[..., : nb * bt, :].reshape(*lead, nb, bt, d)
    return numerics.round_to_f16(blocks.sum(axis=-2) / bt)


def residual_score(rule, features, fc1_w, fc1_b, fc2_w, fc2_b, alpha=1.0):
    """s_j = rule_j + alpha * MLP(features_j) (IntentKV §4, residual).

    A two-layer GELU MLP.  With fc2 initialised to zero the residual is zero
    and the score is the rule score exactly (IntentKV §4 minimum check 2).
    """
    x = np.asarray(features, dtype=np.float64) @ np.asarray(fc1_w, dtype=np.float64).T + fc1_b
    gelu = 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))
    r = gelu @ np.asarray(fc2_w, dtype=np.float64).T + fc2_b
    return np.asarray(rule, dtype=np.float64) + alpha * r[..., 0]


def decode_recovery_step(state, n_seen, q, lse, k_pool, block_table, n_ctx, *,
                         req=None, scale=None):
    """One decode step of the recovery-based action scorer.

    ActKV §7.1 and its Algorithm 3: for the current query token of every
    request that is generating an action, each cached key j of KV head g gets
    p[h,j] = exp(s[h,j] - LSE[h]) for the query heads h of g's group, where
    s = scale * q_h . k_j is recomputed from the paged keys and LSE is the
    log-sum-exp the paged attention pass produced.  The probabilities are
    reduced by a maximum over the group and folded into a running mean over
    the action tokens of the current region; the mean restarts from zero when
    a region begins.

    Readings where the page is silent: the token sees the first n_ctx[r]
    logical positions of its request; positions it cannot see (j >= n_ctx,
    or a block-table entry outside the pool) count as probability 0, so the
    running mean after T tokens equals the plain mean over those T tokens.
    n_seen[r] is the number of action tokens of the region already in the
    state; n_seen == 0 starts a region (the old state is not read).  The
    update for t = n_seen is  state <- state + (p - state) / (t + 1)  over
    every position j < n_cap.

    state: [L][R][Hkv][n_cap]; q: [L][Ra][Hq][D]; lse: [L][Ra][Hq];
    k_pool: [L][P][BS][Hkv][D]; block_table: [R][Y]; n_ctx, n_seen: [R];
    req: [Ra] request of each query row (default 0..R-1).  Returns the new
    state (float64); requests not in ``req`` are unchanged.
    """
    st = np.array(state, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    L, Ra, Hq, D = q.shape
    _, P, BS, Hkv, _ = k_pool.shape
    n_cap = st.shape[3]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    req = np.arange(Ra) if req is None else np.asarray(req, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    j = np.arange(n_cap)
    for a in range(Ra):
        r = int(req[a])
        t = int(n_seen[r])
        n = int(n_ctx[r])
        lp = j // BS
        page = np.where(lp < bt.shape[1], bt[r, np.minimum(lp, bt.shape[1] - 1)], -1)
        visible = (j < n) & (page >= 0) & (page < P)
        pg = np.where(visible, page, 0)
        for l in range(L):
            keys = np.asarray(k_pool[l], dtype=np.float64)[pg, j % BS]      # [n_cap][Hkv][D]
            for g in range(Hkv):
                heads = [h for h in range(Hq) if gqa_group(h, Hq, Hkv) == g]
                probs = [np.exp(scale * (keys[:, g, :] @ q[l, a, h]) - lse[l, a, h]) for h in heads]
                p = np.where(visible, np.max(np.stack(probs), axis=0), 0.0)
                if t == 0:
                    st[l, r, g] = p
                else:
                    st[l, r, g] = st[l, r, g] + (p - st[l, r, g]) / (t + 1)
    return st
