"""Calls at the largest sizes one launch allows: 65535 selection units, 65535
window-score units (layers x KV heads), 65535 requests for the ActKV decode
scorer, the keep score and the compaction.  Sampled rows are compared with the oracle to the
usual bar; invariants are checked for every row."""
import math

import numpy as np
import pytest
import torch

from oracle import score as osc, select as osel
from parity import SCORE_RTOL, require_gpu
from test_gpu_actkv_policy import _check_keep, _check_state

import selection_score_amd as kv

pytestmark = pytest.mark.gpu

MAX = 65535


def _sample(rng, n):
    return sorted(set([0, 1, n // 2, n - 2, n - 1] + rng.choice(n, 40, replace=False).tolist()))


def test_select_at_the_unit_limit():
    dev = require_gpu()
    rng = np.random.default_rng(31)
    n, k, n_sink, n_recent = 96, 12, 2, 3
    s = rng.random((MAX, n), dtype=np.float32)
    kept = torch.full((MAX, k), -7, dtype=torch.int32, device=dev)
    nk = torch.zeros(MAX, dtype=torch.int32, device=dev)
    print("limits: select U=%d" % MAX, flush=True)
    kv.select(torch.from_numpy(s).to(dev), kept, k_total=k, n_sink=n_sink, n_recent=n_recent, n_kept=nk)
    torch.cuda.synchronize()
    got = kept.cpu().numpy()
    assert (nk.cpu().numpy() == k).all()
    assert (np.diff(got, axis=1) > 0).all()
    assert (got[:, :n_sink] == np.arange(n_sink)).all()
    assert (got[:, -n_recent:] == np.arange(n - n_recent, n)).all()
    for u in _sample(rng, MAX):
        ok, _ = osel.select_topk(s[u].astype(np.float64), k, n_sink, n_recent)
        np.testing.assert_array_equal(got[u], ok)


def test_window_scores_at_the_unit_limit():
    dev = require_gpu()
    rng = np.random.default_rng(32)
    L, Hq, Hkv, W, N, D = MAX, 2, 1, 1, 8, 64
    q = rng.standard_normal((L, Hq, W, D)).astype(np.float32)
    k = rng.standard_normal((L, Hkv, N, D)).astype(np.float32)
    out = torch.full((L * Hkv, N), float("nan"), device=dev)
    print("limits: window L*Hkv=%d" % (L * Hkv), flush=True)
    kv.score_window(torch.from_numpy(q).to(dev), torch.from_numpy(k).to(dev), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    # every key is seen by the one window row: each unit's scores sum to Hq
    np.testing.assert_allclose(got.sum(axis=1), Hq, rtol=1e-5)
    for l in _sample(rng, L):
        want, _ = osc.window_scores(q[[l]].astype(np.float64), k[[l]].astype(np.float64))
        np.testing.assert_allclose(got[l], want.reshape(N), rtol=SCORE_RTOL, atol=0)


def test_decode_and_keep_score_at_the_request_limit():
    dev = require_gpu()
    rng = np.random.default_rng(33)
    L, R, Hq, Hkv, D, bs, n_cap = 1, MAX, 4, 1, 64, 16, 16
    P = R + 1
    bt = rng.permutation(P)[:R].reshape(R, 1).astype(np.int32)
    n_ctx = rng.integers(1, n_cap + 1, R).astype(np.int32)
    n_seen = np.zeros(R, dtype=np.int32)
    g = torch.Generator().manual_seed(34)
    pool = torch.randn((L, P, bs, Hkv, D), generator=g).to(torch.bfloat16)
    q = torch.randn((L, R, Hq, D), generator=g).to(torch.bfloat16)
    # LSE over each request's visible keys, float32 on the host (the attention
    # pass's output in a real decode)
    keys = pool[0, torch.from_numpy(bt[:, 0]).long(), :, 0, :].float()            # [R][bs][D]
    logits = torch.bmm(q[0].float(), keys.transpose(1, 2).contiguous()) / math.sqrt(D)
    vis = torch.arange(bs)[None, None, :] < torch.from_numpy(n_ctx).long()[:, None, None]
    lse = torch.logsumexp(logits.masked_fill(~vis, float("-inf")), dim=2)[None].contiguous()   # [1][R][Hq]
    state = torch.full((L, R, Hkv, n_cap), float("nan"), device=dev)
    print("limits: decode Ra=%d" % R, flush=True)
    kv.decode_score(q.to(dev), lse.to(dev), pool.to(dev), torch.from_numpy(bt).to(dev),
                    torch.from_numpy(n_ctx).to(dev), torch.from_numpy(n_seen).to(dev), state)
    torch.cuda.synchronize()
    got = state.cpu().numpy()
    assert np.isfinite(got).all()
    rows = _sample(rng, R)
    q64 = q.float().numpy().astype(np.float64)
    want = osc.decode_recovery_step(np.zeros((L, R, Hkv, n_cap)), n_seen, q64[:, rows],
                                    lse.numpy().astype(np.float64)[:, rows], pool.float().numpy().astype(np.float64),
                                    bt, n_ctx, req=rows)
    _check_state(got[:, rows], want[:, rows], "decode at the request limit")

    # keep score over every request, from a seeded state (not the decode's)
    st = (rng.random((L, R, Hkv, n_cap)) ** 3).astype(np.float32)
    ks0 = rng.random((R, n_cap)).astype(np.float32)
    n_len = rng.integers(0, n_cap + 1, R).astype(np.int32)
    ks = torch.from_numpy(ks0.copy()).to(dev)
    attn = torch.empty((R, n_cap), device=dev)
    hit = torch.empty((R, n_cap), dtype=torch.uint8, device=dev)
    print("limits: keep score Rc=%d" % R, flush=True)
    kv.keep_score(torch.from_numpy(st).to(dev), ks, torch.from_numpy(n_len).to(dev), lam=0.5, top_p=0.9,
                  attn_score=attn, hit=hit)
    torch.cuda.synchronize()
    S = len(rows)
    _check_keep(st.astype(np.float64)[:, rows], ks0[rows], n_len[rows], list(range(S)), 0.5, 0.9,
                ks.cpu().numpy()[rows], hit.cpu().numpy()[rows], attn.cpu().numpy()[rows])


def test_compact_at_the_request_limit():
    from oracle import materialise as om
    dev = require_gpu()
    rng = np.random.default_rng(35)
    R, Y, bs, L, Hkv, D = MAX, 2, 16, 2, 1, 64
    N = Y * bs - 5                                         # a partial last block
    P = R * Y + 3
    bt = rng.permutation(P)[: R * Y].reshape(R, Y).astype(np.int32)
    keep = rng.random((R, N)) < 0.4
    g = torch.Generator().manual_seed(36)
    k_pool = torch.randn((L, P, bs, Hkv, D), generator=g).to(torch.bfloat16)
    v_pool = torch.randn((L, P, bs, Hkv, D), generator=g).to(torch.bfloat16)
    kd, vd = k_pool.to(dev), v_pool.to(dev)
    slot_pos = torch.full((R, Y * bs), -7, dtype=torch.int32, device=dev)
    freed = torch.full((R, Y), -7, dtype=torch.int32, device=dev)
    nfr = torch.full((R,), -7, dtype=torch.int32, device=dev)
    print("limits: compact R=%d" % R, flush=True)
    kv.compact(torch.from_numpy(keep.astype(np.uint8)).to(dev), torch.from_numpy(bt).to(dev), kd, vd, slot_pos,
               freed, nfr, block_size=bs)
    torch.cuda.synchronize()
    X = -(-keep.sum(axis=1) // bs)
    np.testing.assert_array_equal(nfr.cpu().numpy(), Y - X)
    sp, fr = slot_pos.cpu().numpy(), freed.cpu().numpy()
    gk, gv = kd.cpu().view(torch.int16).numpy(), vd.cpu().view(torch.int16).numpy()
    k0, v0 = k_pool.view(torch.int16).numpy(), v_pool.view(torch.int16).numpy()
    for r in _sample(rng, R):
        for l in range(L):
            kp, vp, pos, fb = om.tail_compact(keep[r], np.arange(Y), bs, k0[l][bt[r]], v0[l][bt[r]])
            np.testing.assert_array_equal(gk[l][bt[r]], kp)
            np.testing.assert_array_equal(gv[l][bt[r]], vp)
        np.testing.assert_array_equal(sp[r], pos)
        np.testing.assert_array_equal(fr[r, : len(fb)], bt[r][fb])
        assert np.all(fr[r, len(fb):] == -1)
