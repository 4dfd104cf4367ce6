"""GPU parity of the block-level (Mean-K) path: kvsel_score in block mode,
per-unit and tiled kvsel_select over blocks, the raw-K gather with re-RoPE,
and the incremental view update -- at small sizes and at the full 1M- and
10M-token workload sizes (sampled units checked against the oracle)."""
import numpy as np
import pytest
import torch

from oracle import materialise as om
from oracle import numerics
from oracle import score as osc
from oracle import select as osel
from oracle.rope import rope_rotate
from parity import (Conditioning, assert_rope_close, assert_scores_close, block_score_tolerance, boundary_gap,
                    check_selection, f64, qbar_error_bound, require_gpu)

import selection_score_amd as kv
from selection_score_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("S,W,NB,n_begin,n_count,D", [
    (2, 16, 3000, 0, 3000, 128),          # matrix cores
    (1, 7, 5000, 1000, 777, 128),         # ragged tile inside the index
    (4, 32, 1200, 1100, 100, 128),
    (8, 5, 999, 0, 999, 128),             # eight sessions, a partial 16-row MFMA tile
    (3, 9, 1500, 17, 1001, 64),           # D 64: vector ALUs
])
def test_block_scores_match_oracle(S, W, NB, n_begin, n_count, D):
    dev = require_gpu()
    g = torch.Generator(device=dev).manual_seed(NB)
    L, Hq, Hkv = 2, 8, 2
    q = torch.randn((S, L, Hq, W, D), generator=g, device=dev).to(torch.bfloat16)
    mu = (torch.randn((L, Hkv, NB, D), generator=g, device=dev) * 0.3).to(torch.float16)
    out = torch.empty((S, L * Hkv, n_count), dtype=torch.float32, device=dev)
    qbar = torch.empty((S, L, Hkv, D), dtype=torch.float32, device=dev)
    kv.score_block(q, mu, out, n_kv_heads=Hkv, n_begin=n_begin, n_count=n_count, qbar=qbar)
    torch.cuda.synchronize()
    qb = osc.query_reduce(f64(q), Hkv)
    qerr = qbar_error_bound(np.abs(qb), osc.query_reduce(np.abs(f64(q)), Hkv), (Hq // Hkv) * W)
    assert np.all(np.abs(f64(qbar) - qb) <= qerr)
    full = osc.block_scores(qb, f64(mu))
    tol = block_score_tolerance(full, np.abs(qb), f64(mu), 1 / np.sqrt(D), qerr)
    want = full[..., n_begin:n_begin + n_count]
    assert_scores_close(f64(out).reshape(-1, n_count), want.reshape(-1, n_count),
                        extra_tol=tol[..., n_begin:n_begin + n_count])
    # a second tile from the cached q-bar
    out2 = torch.empty((S, L * Hkv, 50), dtype=torch.float32, device=dev)
    kv.score_block(None, mu, out2, n_kv_heads=Hkv, n_begin=NB - 50, n_count=50, qbar=qbar, qbar_valid=True)
    torch.cuda.synchronize()
    assert_scores_close(f64(out2).reshape(-1, 50), full[..., NB - 50:].reshape(-1, 50),
                        extra_tol=tol[..., NB - 50:])


@pytest.mark.parametrize("S,NB,n_begin,n_count", [
    (4, 70000, 0, 65536),                 # whole chunks
    (2, 5000, 1000, 777),                 # ragged last chunk and word, tile inside the index
    (3, 3000, 17, 1001),
    (1, 300, 0, 40),                      # one partial word
])
def test_block_scores_packed_matches_dense(S, NB, n_begin, n_count):
    """The packed output under per-row thresholds: the admission mask marks
    exactly the columns whose dense score is above the row's threshold (NaN:
    all; -0.0 equal to +0.0), and each 256-column chunk starts with the
    admitted dense scores in column order, bit for bit; positions after
    them stay as they were.  The dense scores themselves are held to the
    oracle by test_block_scores_match_oracle."""
    dev = require_gpu()
    g = torch.Generator(device=dev).manual_seed(NB + S)
    L, Hq, Hkv, W, D = 2, 8, 2, 16, 128
    U = L * Hkv
    q = torch.randn((S, L, Hq, W, D), generator=g, device=dev).to(torch.bfloat16)
    mu = (torch.randn((L, Hkv, NB, D), generator=g, device=dev) * 0.3).to(torch.float16)
    dense = torch.empty((S, U, n_count), dtype=torch.float32, device=dev)
    kv.score_block(q, mu, dense, n_kv_heads=Hkv, n_begin=n_begin, n_count=n_count)
    torch.cuda.synchronize()
    d = dense.cpu().numpy().reshape(S * U, n_count)
    rng = np.random.default_rng(NB)
    # thresholds: NaN, below everything, above everything, a tie with a score, quantiles
    thr = np.quantile(d, rng.uniform(0.5, 0.999, S * U), axis=1).diagonal().astype(np.float32)
    thr[0] = np.nan
    if S * U > 3:
        thr[1], thr[2], thr[3] = -1e30, 1e30, d[3, n_count // 2]
    sentinel = -12345.0
    packed = torch.full((S, U, n_count), sentinel, dtype=torch.float32, device=dev)
    n_words = (n_count + 63) // 64
    mask = torch.full((S, U, n_words), -1, dtype=torch.int64, device=dev)
    kv.score_block(q, mu, packed, n_kv_heads=Hkv, n_begin=n_begin, n_count=n_count,
                   admit=torch.from_numpy(thr).to(dev).reshape(S, U), tile_mask=mask)
    torch.cuda.synchronize()
    pk = packed.cpu().numpy().reshape(S * U, n_count)
    words = mask.cpu().numpy().reshape(S * U, n_words).view(np.uint64)
    bits = ((words[:, :, None] >> np.arange(64, dtype=np.uint64)) & np.uint64(1)).astype(bool)
    bits = bits.reshape(S * U, -1)
    assert not bits[:, n_count:].any()
    for r in range(S * U):
        adm = np.ones(n_count, bool) if np.isnan(thr[r]) else d[r] > thr[r]
        np.testing.assert_array_equal(bits[r, :n_count], adm, err_msg="row %d" % r)
        for c0 in range(0, n_count, 256):
            want = d[r, c0:c0 + 256][adm[c0:c0 + 256]]
            got = pk[r, c0:c0 + 256]
            np.testing.assert_array_equal(got[:len(want)].view(np.uint32), want.view(np.uint32))
            assert np.all(got[len(want):] == sentinel)


def _oracle_unit_scores(q, mu, s, u, Hkv):
    """Oracle block scores of one (session, unit) and the float32 error bound
    of the library's arithmetic for each."""
    l, g = divmod(u, Hkv)
    G = q.shape[2] // Hkv
    qs = f64(q[s:s + 1, l:l + 1, g * G:(g + 1) * G])
    qb = osc.query_reduce(qs, 1)                                              # [1][1][1][D]
    qerr = qbar_error_bound(np.abs(qb), osc.query_reduce(np.abs(qs), 1), G * q.shape[3])
    m = f64(mu[l, g])[None, None]
    want = osc.block_scores(qb, m)
    tol = block_score_tolerance(want, np.abs(qb), m, 1 / np.sqrt(qb.shape[-1]), qerr)
    return want[0, 0, 0], tol[0, 0, 0]


@pytest.mark.timeout(900)
def test_kvmem_1m_workload_full_size():
    """64 layers x 8 KV heads x 32768 blocks in the launch sequence the
    benchmark times (query reduction + block scores, the single-launch
    select, the raw-K gather re-RoPEd to contiguous positions).  Every one
    of the 512 units: scores element by element and kept blocks bit for bit
    (or under the near-tie rule); the gathered K and V on 32 bit-exact units
    drawn in a seeded order."""
    dev = require_gpu()
    cfg = wl.CONFIGS["kvmem1m"]
    mu, w, _ = wl.kvmem_index(cfg, dev)
    q = wl.kvmem_queries(cfg, dev, w, 0)[None]
    raw_k, raw_v, offs = wl.kvmem_raw_store(cfg, dev)
    U, NB, k, D, bt = cfg.U, cfg.N, cfg.k, cfg.D, cfg.bt
    scores = torch.empty((1, U, NB), dtype=torch.float32, device=dev)
    qbar = torch.empty((1, cfg.L, cfg.Hkv, D), dtype=torch.float32, device=dev)
    kv.score_block(q, mu, scores, n_kv_heads=cfg.Hkv, qbar=qbar)
    kept = torch.empty((U, k), dtype=torch.int32, device=dev)
    kv.select(scores[0], kept, k_total=k, n_sink=cfg.n_sink, n_recent=cfg.n_recent)
    vk = torch.empty((U, k * bt, D), dtype=torch.bfloat16, device=dev)
    vv = torch.empty_like(vk)
    kv.gather_rerope(raw_k, raw_v, kept, vk, vv, bt=bt, D=D, src_rows=NB * bt, src_offsets=offs,
                     rope="raw", theta=cfg.theta)
    torch.cuda.synchronize()
    kept_h = kept.cpu().numpy()
    cond = Conditioning("kvmem1m")
    exact = []
    for u in range(U):
        want, tol = _oracle_unit_scores(q, mu, 0, u, cfg.Hkv)
        assert_scores_close(f64(scores[0, u])[None], want[None], "unit %d" % u, extra_tol=tol[None])
        s32 = numerics.round_to_f32(want)
        verdict = check_selection(kept_h[u], s32, k, cfg.n_sink, cfg.n_recent, what="unit %d" % u)
        cond.add(verdict, boundary_gap(s32, k, cfg.n_sink, cfg.n_recent))
        if verdict == "exact":
            exact.append(u)
    for u in np.random.default_rng(cfg.seed).permutation(exact)[:32]:
        l, g = divmod(int(u), cfg.Hkv)
        # only the kept blocks, in kept order: raw-mode positions depend on
        # the entry's rank in the view, not on its block id
        sel = torch.from_numpy(kept_h[u]).to(dev)
        buf = l % cfg.raw_layers
        rk = f64(raw_k[buf, g][sel]).reshape(k * bt, D)
        rv = f64(raw_v[buf, g][sel]).reshape(k * bt, D)
        gk, gv = om.gather_view(rk, rv, np.arange(k), bt, rope="raw", theta=cfg.theta)
        assert_rope_close(f64(vk[u]), gk, "unit %d" % u)
        np.testing.assert_array_equal(f64(vv[u]), gv)
        cond.materialised += 1
    print(cond.report(), flush=True)
    assert cond.exact >= 0.8 * U and cond.materialised == min(32, len(exact))
    assert np.all(kept_h[:, 0] == 0) and np.all(kept_h[:, -4:] == np.arange(NB - 4, NB))
    assert np.all(np.diff(kept_h, axis=1) > 0)


@pytest.mark.timeout(900)
def test_kvmem_10m_workload_full_size():
    """312500 blocks per unit scored in 65536-block tiles for 4 sessions,
    tiled top-4096, and the in-place incremental update of each session's
    4096-page view (previous view shares about half its blocks; moved hits
    re-rotated from raw K at their new positions), in the launch sequence
    the benchmark times (tiles after the first scored in the packed form
    under the running sets' admission thresholds; they are also scored
    densely to hold every score to the oracle and each packed row to its
    dense one).  64 (session, unit) views drawn in a seeded order are
    checked against the oracle: their scores over every tile, their kept
    blocks, and on the bit-exact ones the whole updated view (page table,
    re-RoPEd misses and moved hits, V).  Invariants hold for every view."""
    dev = require_gpu()
    cfg = wl.CONFIGS["kvmem10m"]
    S, U, NB, k, D, bt, tile = cfg.S, cfg.U, cfg.N, cfg.k, cfg.D, cfg.bt, cfg.tile
    room = k - cfg.n_sink - cfg.n_recent
    mu, w, planted = wl.kvmem_index(cfg, dev, n_dirs=S, planted=(room, 10.0))
    qs = torch.stack([wl.kvmem_queries(cfg, dev, w, s) for s in range(S)])
    qbar = torch.empty((S, cfg.L, cfg.Hkv, D), dtype=torch.float32, device=dev)
    SU = S * U
    cs = torch.empty((SU, k), dtype=torch.float32, device=dev)
    ci = torch.empty((SU, k), dtype=torch.int32, device=dev)
    cc = torch.zeros(SU, dtype=torch.int32, device=dev)
    kept = torch.empty((SU, k), dtype=torch.int32, device=dev)
    nk = torch.empty(SU, dtype=torch.int32, device=dev)
    tile_out = torch.empty((S, U, tile), dtype=torch.float32, device=dev)
    dense_out = torch.empty((S, U, tile), dtype=torch.float32, device=dev)
    mask = torch.empty((SU, tile // 64), dtype=torch.int64, device=dev)
    admit = torch.empty(SU, dtype=torch.float32, device=dev)
    pick = np.random.default_rng(cfg.seed).permutation(SU)[:62]
    sample = sorted(set([(0, 0), (S - 1, U - 1)] + [divmod(int(i), U) for i in pick]))
    rows = torch.tensor([s * U + u for (s, u) in sample], device=dev)
    sampled_scores = {su: [] for su in sample}
    n_admitted = []
    for b in range(0, NB, tile):
        n = min(tile, NB - b)
        # the benchmark's sequence: the first tile dense, later ones packed
        # under the previous call's admission thresholds
        thr = admit.cpu().numpy()[rows.cpu().numpy()] if b > 0 else None
        kv.score_block(qs if b == 0 else None, mu, tile_out.view(-1)[: S * U * n].view(S, U, n),
                       n_kv_heads=cfg.Hkv, n_begin=b, n_count=n, qbar=qbar, qbar_valid=b > 0,
                       admit=admit.view(S, U) if b > 0 else None,
                       tile_mask=mask.view(-1)[: SU * ((n + 63) // 64)] if b > 0 else None)
        out = tile_out.view(-1)[: S * U * n].view(SU, n)
        tm = mask.view(-1)[: SU * ((n + 63) // 64)].view(SU, -1) if b > 0 else None
        if b > 0:
            # the same tile dense, to hold every score to the oracle and the
            # packed rows to the dense ones
            kv.score_block(None, mu, dense_out.view(-1)[: S * U * n].view(S, U, n), n_kv_heads=cfg.Hkv,
                           n_begin=b, n_count=n, qbar=qbar, qbar_valid=True)
            dense = dense_out.view(-1)[: S * U * n].view(SU, n)
            d, pk = dense[rows].cpu().numpy(), out[rows].cpu().numpy()
            words = tm[rows].cpu().numpy().view(np.uint64)
            bits = ((words[:, :, None] >> np.arange(64, dtype=np.uint64)) & np.uint64(1)).astype(bool)
            bits = bits.reshape(len(sample), -1)[:, :n]
            for i in range(len(sample)):
                adm = np.ones(n, bool) if np.isnan(thr[i]) else d[i] > thr[i]
                np.testing.assert_array_equal(bits[i], adm)
                for c0 in range(0, n, 256):
                    want = d[i, c0:c0 + 256][adm[c0:c0 + 256]]
                    np.testing.assert_array_equal(pk[i, c0:c0 + len(want)].view(np.uint32), want.view(np.uint32))
            n_admitted.append(int(bits.sum()))
        else:
            dense = out
        kv.select(out, kept, k_total=k, n_sink=cfg.n_sink, n_recent=cfg.n_recent, n_total=NB, base=b,
                  cand_score=cs, cand_idx=ci, cand_count=cc, finalize=b + n == NB, n_kept=nk,
                  tile_mask=tm, admit=admit if b + n < NB else None)
        for (s, u) in sample:
            sampled_scores[(s, u)].append(f64(dense[s * U + u]))
    torch.cuda.synchronize()
    print("admitted per later tile over the sampled views: %s of %d columns" % (n_admitted, len(sample) * tile),
          flush=True)
    kept_h = kept.cpu().numpy()
    assert np.all(nk.cpu().numpy() == k)
    assert len(sample) >= 63
    verdicts = {}
    cond = Conditioning("kvmem10m")
    for (s, u) in sample:
        got = np.concatenate(sampled_scores[(s, u)])
        want, mag = _oracle_unit_scores(qs, mu, s, u, cfg.Hkv)
        assert_scores_close(got[None], want[None], "session %d unit %d" % (s, u), extra_tol=mag[None])
        s32 = numerics.round_to_f32(want)
        verdicts[(s, u)] = (check_selection(kept_h[s * U + u], s32, k, cfg.n_sink, cfg.n_recent,
                                            what="session %d unit %d" % (s, u)), s32)
        cond.add(verdicts[(s, u)][0], boundary_gap(s32, k, cfg.n_sink, cfg.n_recent))
    del tile_out, cs, ci

    # ---- incremental view update
    raw_k = torch.empty((cfg.Hkv, NB, bt, D), dtype=torch.bfloat16, device=dev)
    raw_v = torch.empty_like(raw_k)
    gen = torch.Generator(device=dev).manual_seed(77)
    for h in range(cfg.Hkv):
        raw_k[h].normal_(generator=gen)
        raw_v[h].normal_(generator=gen)
    offs = torch.tensor([((i % U) % cfg.Hkv) * NB * bt * D for i in range(SU)], dtype=torch.int64,
                        device=dev)
    rng = np.random.default_rng(5)
    prev_idx = np.empty((SU, k), np.int32)
    prev_page = np.empty((SU, k), np.int32)
    planted_h = planted.cpu().numpy()                        # [S][L][Hkv][room]
    for i in range(SU):
        s, u = divmod(i, U)
        l, g = divmod(u, cfg.Hkv)
        inside = rng.choice(planted_h[s, l, g], k // 2, replace=False)
        taken = np.zeros(NB, bool)
        taken[planted_h[s, l, g]] = True
        draw = np.unique(rng.integers(0, NB, 3 * k))
        draw = draw[~taken[draw]]
        outside = rng.choice(draw, k - k // 2, replace=False)
        prev_idx[i] = np.sort(np.concatenate([inside, outside]))
        prev_page[i] = rng.permutation(k)
    pool_k = torch.full((SU, k, bt, D), 0.5, dtype=torch.bfloat16, device=dev)
    pool_v = torch.full((SU, k, bt, D), -0.25, dtype=torch.bfloat16, device=dev)
    o = np.arange(bt)
    baked = {}
    for (s, u) in sample:                                    # sampled views hold real baked K
        verdict, s32 = verdicts[(s, u)]
        if verdict != "exact":
            continue
        i = s * U + u
        g = u % cfg.Hkv
        new_idx, _ = osel.select_topk(s32, k, cfg.n_sink, cfg.n_recent)
        # only the blocks the update touches, renumbered by rank (order kept)
        need = np.union1d(prev_idx[i], new_idx)
        sel = torch.from_numpy(need).to(dev)
        rk, rv = f64(raw_k[g][sel]), f64(raw_v[g][sel])
        prev_r = np.searchsorted(need, prev_idx[i])
        new_r = np.searchsorted(need, new_idx)
        # the previous view: hits baked at their old positions (pages the
        # update overwrites keep the synthetic fill; the oracle reads them too)
        pk = np.full((k, bt, D), 0.5)
        pv = np.full((k, bt, D), -0.25)
        hit = np.isin(prev_idx[i], new_idx)
        for j in np.flatnonzero(hit):
            b = prev_r[j]
            pk[prev_page[i, j]] = numerics.round_to_bf16(rope_rotate(rk[b], j * bt + o, cfg.theta))
            pv[prev_page[i, j]] = rv[b]
        pool_k[i] = torch.from_numpy(pk.astype(np.float32)).to(torch.bfloat16).to(dev)
        pool_v[i] = torch.from_numpy(pv.astype(np.float32)).to(torch.bfloat16).to(dev)
        baked[(s, u)] = (pk, pv, rk, rv, prev_r, new_r)
    pt = torch.empty((SU, k), dtype=torch.int32, device=dev)
    nm = torch.empty(SU, dtype=torch.int32, device=dev)
    kv.gather_incremental(raw_k, raw_v, kept, torch.from_numpy(prev_idx).to(dev),
                          torch.from_numpy(prev_page).to(dev), pool_k, pool_v, pt, nm, bt=bt, D=D,
                          src_rows=NB * bt, src_offsets=offs, rope="raw", theta=cfg.theta, hit_raw=True)
    torch.cuda.synchronize()
    pt_h, nm_h = pt.cpu().numpy(), nm.cpu().numpy()
    assert 0.4 * k < nm_h.mean() < 0.6 * k                 # about half the view is new
    assert np.all(np.sort(pt_h, axis=1) == np.arange(k))   # each page used once per view
    for (s, u), (pk, pv, rk, rv, prev_r, new_r) in baked.items():
        i = s * U + u
        ok, ov, opt, onm = om.incremental_view(prev_r, prev_page[i], new_r, pk, pv, rk, rv, bt,
                                               theta=cfg.theta, hits="raw")
        assert nm_h[i] == onm
        np.testing.assert_array_equal(pt_h[i], opt)
        np.testing.assert_array_equal(f64(pool_v[i]), ov)
        assert_rope_close(f64(pool_k[i]), ok, "session %d unit %d" % (s, u))
        cond.materialised += 1
    print(cond.report(), flush=True)
    assert cond.exact >= 0.8 * len(sample) and cond.materialised == cond.exact
