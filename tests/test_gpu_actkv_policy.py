"""GPU parity of ActKV's decode-streaming recovery scorer (kvsel_decode_score)
and LRFU keep score (kvsel_keep_score) against the oracle.

Acceptance:
  * scorer state: |gpu - oracle| <= 1e-4 * |oracle| + 1e-30 element-wise.
    The probabilities come from bf16/f16 logits accumulated in float32 and
    one exp2, so their relative error is a few 1e-6; a wrong head, position,
    group or mean weight is off by far more;
  * action scores: bit-exact (both sides round an exact or compensated
    float64 sum of the same float32 state once to float32);
  * hits: bit-exact, except that the boundary of the top-p prefix may move
    where the oracle's float64 cumulative sum lies within 1e-12 * total of
    the target (different summation orders); the GPU set must then still be
    a prefix of the oracle's order whose sum reaches the target within that
    band;
  * keep scores: within 1 float32 ulp of lambda * KS + hit * score (the GPU
    fuses the multiply-add; the oracle rounds its float64 result once).
"""
import math

import numpy as np
import pytest
import torch

from oracle import paging, score as osc, select as osel
from parity import require_gpu

import selection_score_amd as kv
from selection_score_amd import workloads as wl

pytestmark = pytest.mark.gpu

STATE_RTOL = 1e-4
CUM_BAND = 1e-12


def _f64(t):
    return t.detach().cpu().float().numpy().astype(np.float64)


def _true_lse(q, k_pool, bt, n_ctx, BS, G):
    """float64 log-sum-exp of scale * q . k over each request's visible keys
    (what a paged attention pass returns, here exact)."""
    L, Ra, Hq, D = q.shape
    Hkv = k_pool.shape[3]
    P = k_pool.shape[1]
    out = np.zeros((L, Ra, Hq))
    for a in range(Ra):
        n = int(n_ctx[a])
        j = np.arange(n)
        page = bt[a, j // BS]
        vis = (page >= 0) & (page < P)
        for l in range(L):
            keys = k_pool[l][np.where(vis, page, 0), j % BS]          # [n][Hkv][D]
            for h in range(Hq):
                s = keys[:, h // G, :] @ q[l, a, h] / math.sqrt(D)
                s = s[vis]
                m = s.max() if s.size else 0.0
                out[l, a, h] = m + math.log(max(np.sum(np.exp(s - m)), 1e-300))
    return out


def _check_state(got, want, what):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    nan_w = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan_w), what + ": NaN pattern differs"
    g, w = got[~nan_w], want[~nan_w]
    bad = np.abs(g - w) > STATE_RTOL * np.abs(w) + 1e-30
    if bad.any():
        i = int(np.argmax(bad))
        raise AssertionError("%s: %d of %d out of tolerance; first gpu %r oracle %r"
                             % (what, int(bad.sum()), bad.size, g[i], w[i]))


def _decode_case(dev, *, L, R, Ra, Hq, Hkv, D, BS, n_cap, n_ctx_steps, req, dtype, T, seed, bad_blocks=0):
    """Stream T decode tokens through the GPU and the oracle; compare the
    state after every token."""
    rng = np.random.default_rng(seed)
    G = Hq // Hkv
    Y = -(-n_cap // BS)
    P = R * Y + 5
    bt = rng.permutation(P)[: R * Y].reshape(R, Y).astype(np.int32)
    for _ in range(bad_blocks):                       # entries outside the pool score 0
        bt[rng.integers(R), rng.integers(Y)] = rng.choice([-1, P, P + 100])
    tdt = dtype
    k_pool = torch.randn((L, P, BS, Hkv, D), generator=torch.Generator().manual_seed(seed)).to(tdt)
    k64 = _f64(k_pool)
    kd = k_pool.to(dev)
    btd = torch.from_numpy(bt).to(dev)
    reqd = None if req is None else torch.tensor(req, dtype=torch.int32, device=dev)
    rows = list(range(Ra)) if req is None else list(req)
    state0 = np.full((L, R, Hkv, n_cap), np.nan)       # a region start must not read it
    st_gpu = torch.from_numpy(state0.astype(np.float32)).to(dev)
    st_ora = state0.copy()
    for t in range(T):
        n_ctx = np.array(n_ctx_steps[t], dtype=np.int32)
        n_seen = np.full(R, t, dtype=np.int32)
        q = torch.randn((L, Ra, Hq, D), generator=torch.Generator().manual_seed(seed * 100 + t)) * 1.5
        q = q.to(tdt)
        q64 = _f64(q)
        lse = _true_lse(q64, k64, bt[rows], np.minimum(n_ctx[rows], n_cap), BS, G).astype(np.float32)
        print("decode step %d L%d R%d Ra%d Hq%d Hkv%d D%d BS%d n_cap%d %s" % (t, L, R, Ra, Hq, Hkv, D, BS, n_cap, dtype),
              flush=True)
        kv.decode_score(q.to(dev), torch.from_numpy(lse).to(dev), kd, btd, torch.from_numpy(n_ctx).to(dev),
                        torch.from_numpy(n_seen).to(dev), st_gpu, req=reqd)
        torch.cuda.synchronize()
        st_ora = osc.decode_recovery_step(st_ora, n_seen, q64, lse.astype(np.float64), k64, bt, n_ctx,
                                          req=rows)
        _check_state(st_gpu.cpu().numpy(), st_ora, "state after token %d" % t)
    return st_gpu, st_ora


@pytest.mark.parametrize("Hq,Hkv,D,dtype", [(32, 8, 128, torch.bfloat16), (16, 2, 128, torch.float16),
                                            (8, 8, 64, torch.bfloat16), (12, 4, 64, torch.float16),
                                            (16, 1, 128, torch.bfloat16)])
def test_decode_stream_matches_oracle(Hq, Hkv, D, dtype):
    # 3 of 5 requests generate actions; ragged contexts crossing 64-position
    # tiles and 16-slot blocks; the context grows by one per token
    dev = require_gpu()
    n0 = np.array([150, 1, 64, 200, 77])
    steps = [np.minimum(n0 + t, 203) for t in range(3)]
    _decode_case(dev, L=2, R=5, Ra=3, Hq=Hq, Hkv=Hkv, D=D, BS=16, n_cap=203, n_ctx_steps=steps,
                 req=[4, 0, 2], dtype=dtype, T=3, seed=Hq + D)


def test_decode_block32_unmapped_blocks_and_identity_rows():
    dev = require_gpu()
    n0 = np.array([300, 0, 129, 256])
    steps = [n0 + t for t in range(2)]
    _decode_case(dev, L=3, R=4, Ra=4, Hq=32, Hkv=8, D=128, BS=32, n_cap=320, n_ctx_steps=steps, req=None,
                 dtype=torch.bfloat16, T=2, seed=5, bad_blocks=3)


def test_decode_full_size_sampled_rows():
    # one decode token of all 64 requests at 6144 positions, 36 layers, 8 KV
    # heads, 32 query heads, mid-region (5 tokens already in the state); the
    # oracle recomputes sampled (layer, request, KV head) rows
    dev = require_gpu()
    cfg = wl.CONFIGS["actkv"]
    inp = wl.actkv_decode_inputs(cfg, dev)
    state = wl.actkv_state(cfg, dev)
    rng = np.random.default_rng(3)
    picks = [(int(rng.integers(cfg.L)), int(rng.integers(cfg.S)), int(rng.integers(cfg.Hkv))) for _ in range(6)]
    picks += [(0, 0, 0), (cfg.L - 1, cfg.S - 1, cfg.Hkv - 1)]
    before = {p: state[p].cpu().numpy().astype(np.float64) for p in picks}
    print("decode full size", flush=True)
    kv.decode_score(inp["q"], inp["lse"], inp["k_pool"], inp["block_table"], inp["n_ctx"], inp["n_seen"], state)
    torch.cuda.synchronize()
    bs, G = cfg.page_size, cfg.G
    t = cfg.turns
    for (l, r, g) in picks:
        bt = inp["block_table"][r].cpu().numpy()
        keys = inp["k_pool"][l][inp["block_table"][r].long()].cpu()      # [Y][bs][Hkv][D]
        k1 = _f64(keys[:, :, g:g + 1])[None]                             # one KV head, identity block table
        q1 = _f64(inp["q"][l, r, g * G:(g + 1) * G])[None, None]
        lse1 = _f64(inp["lse"][l, r, g * G:(g + 1) * G])[None, None]
        st1 = before[(l, r, g)][None, None, None]
        want = osc.decode_recovery_step(st1, [t], q1, lse1, k1, np.arange(len(bt))[None], [cfg.N])
        _check_state(state[l, r, g].cpu().numpy(), want[0, 0, 0], "row %s" % ((l, r, g),))


# ---------------------------------------------------------------- keep score

def _check_keep(state64, ks0, n_len, req, lam, top_p, ks_gpu, hit_gpu, attn_gpu):
    R, n_cap = ks0.shape
    lam = float(np.float32(lam))
    top_p = float(np.float32(top_p))
    near = 0
    for r in range(R):
        if r not in set(req):
            np.testing.assert_array_equal(ks_gpu[r], ks0[r])
            continue
        n = int(min(max(n_len[r], 0), n_cap))
        a = osel.action_scores(state64, r, n)
        np.testing.assert_array_equal(attn_gpu[r, :n], a.astype(np.float32))
        assert not attn_gpu[r, n:].any() and not hit_gpu[r, n:].any()
        np.testing.assert_array_equal(ks_gpu[r, n:], ks0[r, n:])
        h_ora = osel.top_p_hits(a, top_p)
        h = hit_gpu[r, :n].astype(bool)
        if not np.array_equal(h, h_ora):
            # the prefix boundary may only move inside the rounding band
            order = np.lexsort((np.arange(n), -a))
            cum = np.cumsum(a[order])
            target = top_p * cum[-1]
            m = int(h.sum())
            assert np.array_equal(np.sort(order[:m]), np.nonzero(h)[0]), "request %d: hits are not a prefix" % r
            assert cum[m - 1] >= target - CUM_BAND * cum[-1], r
            assert m == 1 or cum[m - 2] < target + CUM_BAND * cum[-1], r
            near += 1
        want = lam * ks0[r, :n] + np.where(h, a, 0.0)
        got = ks_gpu[r, :n].astype(np.float64)
        ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(got - want) <= ulp), "request %d keep score" % r
    return near


def _keep_case(dev, state, ks0, n_len, req, lam, top_p, with_outputs=True):
    L, R, Hkv, n_cap = state.shape
    sd = torch.from_numpy(state.astype(np.float32)).to(dev)
    ksd = torch.from_numpy(ks0.astype(np.float32)).to(dev)
    attn = torch.full((R, n_cap), -7.0, device=dev)
    hit = torch.full((R, n_cap), 7, dtype=torch.uint8, device=dev)
    reqd = None if req is None else torch.tensor(req, dtype=torch.int32, device=dev)
    print("keep score L%d R%d Hkv%d n_cap%d req %s lam %g top_p %g" % (L, R, Hkv, n_cap, req, lam, top_p),
          flush=True)
    kv.keep_score(sd, ksd, torch.tensor(n_len, dtype=torch.int32, device=dev), lam=lam, top_p=top_p, req=reqd,
                  attn_score=attn if with_outputs else None, hit=hit if with_outputs else None)
    torch.cuda.synchronize()
    return ksd.cpu().numpy(), hit.cpu().numpy(), attn.cpu().numpy()


@pytest.mark.parametrize("lam,top_p", [(0.5, 0.9), (0.0, 0.9), (1.0, 0.3), (0.25, 1.0)])
def test_keep_score_matches_oracle(lam, top_p):
    dev = require_gpu()
    rng = np.random.default_rng(int(lam * 100 + top_p * 10))
    L, R, Hkv, n_cap = 3, 6, 4, 2500
    state = (rng.random((L, R, Hkv, n_cap)) ** 6 * rng.random((1, R, 1, 1))).astype(np.float32).astype(np.float64)
    state[:, 3] = 0.0                                     # a request with no attention: no hits
    ks0 = (rng.random((R, n_cap)) * 0.01).astype(np.float32).astype(np.float64)
    n_len = np.array([2500, 1, 2047, 1500, 0, 1025])
    req = [5, 0, 2, 3, 1, 4] if lam != 1.0 else [2, 5]
    ks, hit, attn = _keep_case(dev, state, ks0, n_len, req, lam, top_p)
    near = _check_keep(state, ks0, n_len, req, lam, top_p, ks, hit, attn)
    assert near <= 1


def test_keep_score_ties_resolve_by_index():
    # every entry has the same score: exactly ceil(top_p * n) entries, the
    # lowest indices, are hit (ranked across several 1024-entry chunks)
    dev = require_gpu()
    L, R, Hkv, n_cap = 2, 3, 2, 3000
    state = np.full((L, R, Hkv, n_cap), 1.0 / 64)
    state[:, 2, :, ::3] = 1.0 / 32                       # request 2: two levels, ties in each
    ks0 = np.zeros((R, n_cap))
    n_len = np.array([3000, 2999, 3000])
    ks, hit, attn = _keep_case(dev, state, ks0, n_len, None, 0.5, 0.5)
    assert hit[0].sum() == 1500 and hit[0, :1500].all()
    assert hit[1].sum() == 1500 and hit[1, :1500].all()
    assert _check_keep(state, ks0, n_len, [0, 1, 2], 0.5, 0.5, ks, hit, attn) == 0


def test_keep_score_without_optional_outputs():
    dev = require_gpu()
    rng = np.random.default_rng(8)
    L, R, Hkv, n_cap = 2, 4, 2, 777
    state = (rng.random((L, R, Hkv, n_cap)) ** 4).astype(np.float32).astype(np.float64)
    ks0 = rng.random((R, n_cap)).astype(np.float32).astype(np.float64)
    n_len = np.array([777, 500, 3, 776])
    ks_a, hit, attn = _keep_case(dev, state, ks0, n_len, [1, 3], 0.75, 0.9)
    ks_b, _, _ = _keep_case(dev, state, ks0, n_len, [1, 3], 0.75, 0.9, with_outputs=False)
    np.testing.assert_array_equal(ks_a, ks_b)
    _check_keep(state, ks0, n_len, [1, 3], 0.75, 0.9, ks_a, hit, attn)


def test_keep_score_full_size_sampled_requests():
    dev = require_gpu()
    cfg = wl.CONFIGS["actkv"]
    state = wl.actkv_state(cfg, dev)
    R, N = cfg.S, cfg.N
    ks = torch.rand((R, N), generator=torch.Generator(device=dev).manual_seed(4), device=dev) * 1e-3
    ks0 = ks.cpu().numpy().astype(np.float64)
    attn = torch.empty((R, N), device=dev)
    hit = torch.empty((R, N), dtype=torch.uint8, device=dev)
    n_len = torch.full((R,), N, dtype=torch.int32, device=dev)
    print("keep score full size", flush=True)
    kv.keep_score(state, ks, n_len, lam=cfg.decay, top_p=0.9, attn_score=attn, hit=hit)
    torch.cuda.synchronize()
    ks_g, hit_g, attn_g = ks.cpu().numpy(), hit.cpu().numpy(), attn.cpu().numpy()
    for r in (0, 17, 40, R - 1):
        st_r = state[:, r:r + 1].cpu().numpy().astype(np.float64)
        sub = _check_keep(st_r, ks0[r:r + 1], [N], [0], cfg.decay, 0.9, ks_g[r:r + 1], hit_g[r:r + 1],
                          attn_g[r:r + 1])
        assert sub <= 1
        frac = hit_g[r].mean()
        assert 0.05 < frac < 0.95, frac                  # the top-p set is a real subset here


def test_decode_edges_many_heads_clamps_and_skipped_rows():
    # 16 KV heads (the workgroup loops over heads), an explicit scale, a
    # request list with an out-of-range entry (skipped), n_ctx beyond the
    # state and the block table (clamped), and a negative token count (a
    # region start)
    dev = require_gpu()
    rng = np.random.default_rng(21)
    L, R, Hq, Hkv, D, BS, n_cap = 2, 3, 32, 16, 64, 16, 100
    G = Hq // Hkv
    Y = 7                                                # 112 slots >= n_cap
    P = R * Y + 2
    bt = rng.permutation(P)[: R * Y].reshape(R, Y).astype(np.int32)
    k_pool = torch.randn((L, P, BS, Hkv, D), generator=torch.Generator().manual_seed(2)).to(torch.bfloat16)
    k64 = _f64(k_pool)
    q = (torch.randn((L, 3, Hq, D), generator=torch.Generator().manual_seed(3)) * 2).to(torch.bfloat16)
    q64 = _f64(q)
    req = [2, 7, 0]                                      # row 1 names no request
    n_ctx = np.array([500, 40, 60], dtype=np.int32)      # request 0 clamps to n_cap
    n_seen = np.array([-3, 0, 2], dtype=np.int32)
    scale = 0.3
    lse = np.zeros((L, 3, Hq), dtype=np.float32)
    for a, r in enumerate(req):
        if r >= R:
            lse[:, a] = 1.0
            continue
        n = min(int(n_ctx[r]), n_cap)
        sm = paging.slot_map_from_block_table(bt[r], BS, n)
        for l in range(L):
            k = paging.logical_keys_from_pool(k64[l], sm, BS)
            for h in range(Hq):
                s = scale * (k[h // G] @ q64[l, a, h])
                lse[l, a, h] = np.log(np.sum(np.exp(s - s.max()))) + s.max()
    state0 = rng.random((L, R, Hkv, n_cap)).astype(np.float32)
    state0[:, 2, :, 60:] = 0.0                           # request 2 is mid-region: zeros past its context
    st = torch.from_numpy(state0.copy()).to(dev)
    print("decode edges", flush=True)
    kv.decode_score(q.to(dev), torch.from_numpy(lse).to(dev), k_pool.to(dev), torch.from_numpy(bt).to(dev),
                    torch.from_numpy(n_ctx).to(dev), torch.from_numpy(n_seen).to(dev), st,
                    req=torch.tensor(req, dtype=torch.int32, device=dev), scale=scale)
    torch.cuda.synchronize()
    rows = [2, 0]
    want = osc.decode_recovery_step(state0.astype(np.float64), np.maximum(n_seen, 0), q64[:, [0, 2]],
                                    lse[:, [0, 2]].astype(np.float64), k64, bt, np.minimum(n_ctx, n_cap),
                                    req=rows, scale=scale)
    _check_state(st.cpu().numpy(), want, "edges")
    np.testing.assert_array_equal(st[:, 1].cpu().numpy(), state0[:, 1])    # untouched request


def test_keep_score_long_rows_odd_stride_and_misaligned_state():
    # 100003 positions (the row stride is not a multiple of 4 and the state
    # starts 4 bytes past a 16-byte boundary: the scalar load path), n_len
    # past n_cap (clamped), 98 chunks of 1024 entries in the update pass
    dev = require_gpu()
    rng = np.random.default_rng(31)
    L, R, Hkv, n_cap = 2, 2, 2, 100003
    vals = (rng.random((L, R, Hkv, n_cap)) ** 8).astype(np.float32)
    flat = torch.zeros(vals.size + 1, dtype=torch.float32, device=dev)
    flat[1:] = torch.from_numpy(vals.reshape(-1)).to(dev)
    sd = flat[1:].view(L, R, Hkv, n_cap)
    assert sd.data_ptr() % 16 == 4
    ks0 = (rng.random((R, n_cap)) * 1e-3).astype(np.float32)
    ksd = torch.from_numpy(ks0.copy()).to(dev)
    attn = torch.empty((R, n_cap), device=dev)
    hit = torch.empty((R, n_cap), dtype=torch.uint8, device=dev)
    n_len = [200000, 70001]
    print("keep score long rows", flush=True)
    kv.keep_score(sd, ksd, torch.tensor(n_len, dtype=torch.int32, device=dev), lam=0.5, top_p=0.9,
                  attn_score=attn, hit=hit)
    torch.cuda.synchronize()
    near = _check_keep(vals.astype(np.float64), ks0.astype(np.float64), n_len, [0, 1], 0.5, 0.9,
                       ksd.cpu().numpy(), hit.cpu().numpy(), attn.cpu().numpy())
    assert near <= 1


def test_compression_pipeline_decode_keep_select_compact():
    # ActKV's chain on the GPU: three decode tokens of an action region, the
    # LRFU keep score at the region's end, eviction to a budget by keep
    # score, and the in-place tail compaction of K and V.  The oracle runs
    # the same chain; the data has no near-ties, so the keep masks, slot maps
    # and pools must agree exactly
    from oracle import materialise as om
    dev = require_gpu()
    rng = np.random.default_rng(41)
    L, R, Hq, Hkv, D, BS, N, T = 2, 3, 8, 2, 64, 16, 160, 3
    G = Hq // Hkv
    Y = N // BS
    P = R * Y + 4
    k_total, n_sink, n_recent, lam, top_p = 96, 4, 16, 0.5, 0.9
    bt = rng.permutation(P)[: R * Y].reshape(R, Y).astype(np.int32)
    gk = torch.Generator().manual_seed(42)
    k_pool = torch.randn((L, P, BS, Hkv, D), generator=gk).to(torch.bfloat16)
    v_pool = torch.randn((L, P, BS, Hkv, D), generator=gk).to(torch.bfloat16)
    k64 = _f64(k_pool)
    n_ctx = np.full(R, N, dtype=np.int32)
    kd, vd, btd = k_pool.to(dev), v_pool.to(dev), torch.from_numpy(bt).to(dev)
    st_gpu = torch.zeros((L, R, Hkv, N), device=dev)
    st_ora = np.zeros((L, R, Hkv, N))
    for t in range(T):
        q = (torch.randn((L, R, Hq, D), generator=torch.Generator().manual_seed(50 + t)) * 2).to(torch.bfloat16)
        q64 = _f64(q)
        lse = _true_lse(q64, k64, bt, n_ctx, BS, G).astype(np.float32)
        n_seen = np.full(R, t, dtype=np.int32)
        kv.decode_score(q.to(dev), torch.from_numpy(lse).to(dev), kd, btd, torch.from_numpy(n_ctx).to(dev),
                        torch.from_numpy(n_seen).to(dev), st_gpu)
        st_ora = osc.decode_recovery_step(st_ora, n_seen, q64, lse.astype(np.float64), k64, bt, n_ctx)
    ks0 = (rng.random((R, N)) * 0.02).astype(np.float32)
    ks_gpu = torch.from_numpy(ks0.copy()).to(dev)
    kv.keep_score(st_gpu, ks_gpu, torch.from_numpy(n_ctx).to(dev), lam=lam, top_p=top_p)
    kept = torch.empty((R, k_total), dtype=torch.int32, device=dev)
    keep = torch.empty((R, N), dtype=torch.uint8, device=dev)
    kv.select(ks_gpu, kept, k_total=k_total, n_sink=n_sink, n_recent=n_recent, keep_mask=keep)
    slot_pos = torch.empty((R, Y * BS), dtype=torch.int32, device=dev)
    freed = torch.empty((R, Y), dtype=torch.int32, device=dev)
    nfr = torch.empty(R, dtype=torch.int32, device=dev)
    print("actkv pipeline", flush=True)
    kv.compact(keep, btd, kd, vd, slot_pos, freed, nfr, block_size=BS)
    torch.cuda.synchronize()

    ks_ora, _, _ = osel.keep_score_step(st_ora, ks0.astype(np.float64), n_ctx, lam=lam,
                                        top_p=float(np.float32(top_p)))
    for r in range(R):
        # the top-p boundary is also well clear: the GPU's running means differ
        # from the oracle's by ~1e-6 relative, far below this margin
        a = osel.action_scores(st_ora, r, N)
        cum = np.cumsum(np.sort(a)[::-1])
        target = float(np.float32(top_p)) * cum[-1]
        m = int(np.searchsorted(cum, target)) + 1
        assert cum[m - 1] - target > 1e-4 * cum[-1] and target - cum[m - 2] > 1e-4 * cum[-1]
    ks32 = ks_ora.astype(np.float32).astype(np.float64)
    np.testing.assert_allclose(ks_gpu.cpu().numpy(), ks32, rtol=1e-4, atol=0)
    want_k, want_v = k_pool.clone(), v_pool.clone()
    for r in range(R):
        idx, mask = osel.select_topk(ks32[r], k_total, n_sink, n_recent)
        # the oracle's boundary is well clear of ties, so the GPU's keep
        # scores (within 1e-4) must pick the same set
        cand = np.sort(ks32[r][n_sink:N - n_recent])[::-1]
        room = k_total - n_sink - n_recent
        assert (cand[room - 1] - cand[room]) > 1e-4 * cand[room - 1], (r, cand[room - 1], cand[room])
        np.testing.assert_array_equal(keep[r].cpu().numpy().astype(bool), mask)
        np.testing.assert_array_equal(kept[r].cpu().numpy(), idx)
        for l in range(L):
            kp, vp, pos, fb = om.tail_compact(mask, bt[r], BS, want_k[l].view(torch.int16).numpy(),
                                              want_v[l].view(torch.int16).numpy())
            want_k[l] = torch.from_numpy(kp).view(torch.bfloat16)
            want_v[l] = torch.from_numpy(vp).view(torch.bfloat16)
        np.testing.assert_array_equal(slot_pos[r].cpu().numpy(), pos)
        assert nfr[r].item() == len(fb)
        np.testing.assert_array_equal(freed[r, : len(fb)].cpu().numpy(), fb)
    assert torch.equal(kd.cpu().view(torch.int16), want_k.view(torch.int16))
    assert torch.equal(vd.cpu().view(torch.int16), want_v.view(torch.int16))
