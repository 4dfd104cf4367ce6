"""GPU parity of window scoring (kvsel_score, window mode) and of the whole
token-level path: score -> pool -> select -> gather."""
import numpy as np
import pytest
import torch

from oracle import materialise as om
from oracle import numerics
from oracle import score as osc
from parity import Conditioning, assert_scores_close, boundary_gap, check_selection, f64, require_gpu

import selection_score_amd as kv
from selection_score_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _window(dev, q, k, **kw):
    L, Hq, W, D = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    out = torch.empty((L * Hkv, N), dtype=torch.float32, device=dev)
    lse = torch.empty((L, Hq, W), dtype=torch.float32, device=dev)
    kv.score_window(q, k, out, lse_out=lse if kw.pop("want_lse", True) else None, **kw)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("dtype,L,Hkv,Hq,W,N,D,causal", [
    (torch.bfloat16, 2, 2, 8, 32, 5000, 128, True),     # MFMA: 3 key chunks, ragged tail, 2 row waves
    (torch.bfloat16, 1, 2, 8, 64, 4096, 128, False),    # MFMA: full 256-row unit, non-causal
    (torch.float16, 1, 1, 4, 16, 2100, 64, True),       # MFMA: D = 64, one row wave
    (torch.float32, 1, 2, 8, 16, 2048, 64, True),       # VALU: float32 (the tiny workload's shape)
    (torch.bfloat16, 2, 2, 4, 3, 777, 128, True),       # VALU: W < 16
])
def test_window_scores_and_lse_match_oracle(dtype, L, Hkv, Hq, W, N, D, causal):
    dev = require_gpu()
    g = torch.Generator(device=dev).manual_seed(N + W)
    q = (torch.randn((L, Hq, W, D), generator=g, device=dev) * 1.5).to(dtype)
    k = (torch.randn((L, Hkv, N, D), generator=g, device=dev) * 1.5).to(dtype)
    out, lse = _window(dev, q, k, causal=causal)
    a, ol = osc.window_scores(f64(q), f64(k), causal=causal)
    assert_scores_close(f64(lse)[None], ol[None], "lse")
    assert_scores_close(f64(out), a.reshape(L * Hkv, N))
    # without an LSE output the vector-ALU score pass merges the LSE partials
    # itself (the combine's arithmetic): the same bits
    out2, _ = _window(dev, q, k, causal=causal, want_lse=False)
    assert torch.equal(out2.view(torch.int32), out.view(torch.int32))


def test_window_lse_recovery_and_aggregations():
    dev = require_gpu()
    g = torch.Generator(device=dev).manual_seed(3)
    L, Hkv, Hq, W, N, D = 1, 2, 8, 64, 3000, 128
    q = torch.randn((L, Hq, W, D), generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn((L, Hkv, N, D), generator=g, device=dev).to(torch.bfloat16)
    qo, ko = f64(q), f64(k)
    _, ol = osc.window_scores(qo, ko)
    lse_in = numerics.round_to_f32(ol + 0.25)             # a caller-supplied LSE
    for head_agg, row_agg in [("sum", "sum"), ("mean", "mean"), ("max", "mean"), ("sum", "max")]:
        out = torch.empty((L * Hkv, N), dtype=torch.float32, device=dev)
        kv.score_window(q, k, out, lse_in=torch.from_numpy(lse_in).to(dev), head_agg=head_agg,
                        row_agg=row_agg)
        torch.cuda.synchronize()
        a, _ = osc.window_scores(qo, ko, lse_in=lse_in.astype(np.float64), head_agg=head_agg,
                                 row_agg=row_agg)
        assert_scores_close(f64(out), a.reshape(L * Hkv, N), "%s/%s" % (head_agg, row_agg))


@pytest.mark.parametrize("pool", ["avg", "max"])
def test_window_pooling(pool):
    dev = require_gpu()
    g = torch.Generator(device=dev).manual_seed(4)
    q = torch.randn((1, 4, 16, 64), generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn((1, 1, 1500, 64), generator=g, device=dev).to(torch.bfloat16)
    out, _ = _window(dev, q, k, pool=pool, pool_k=7, want_lse=False)
    a, _ = osc.window_scores(f64(q), f64(k))
    assert_scores_close(f64(out), osc.pool1d(a, pool, 7).reshape(1, -1))


def _token_path(dev, cfg, inp):
    """score -> select (pooling the scores in its own workgroup) -> gather on
    the GPU, the tiny step's launch sequence; returns host copies."""
    q, k, v = inp["q"], inp["k"], inp["v"]
    U, N = cfg.U, cfg.N
    scores = torch.empty((U, N), dtype=torch.float32, device=dev)
    kv.score_window(q, k, scores)
    kept = torch.empty((U, cfg.k), dtype=torch.int32, device=dev)
    mask = torch.empty((U, N), dtype=torch.uint8, device=dev)
    kv.select(scores, kept, k_total=cfg.k, n_sink=cfg.n_sink, n_recent=cfg.n_recent, keep_mask=mask,
              pool=cfg.pool, pool_k=cfg.pool_k)
    dk = torch.empty((U, cfg.k, cfg.D), dtype=k.dtype, device=dev)
    dv = torch.empty_like(dk)
    kv.gather_rerope(k.view(U, N, cfg.D), v.view(U, N, cfg.D), kept, dk, dv, bt=1, D=cfg.D, src_rows=N,
                     src_unit_stride=N * cfg.D)
    torch.cuda.synchronize()
    return scores, kept, mask, dk, dv


def _oracle_unit(cfg, q, k, u):
    l, g = divmod(u, cfg.Hkv)
    heads = slice(g * cfg.G, (g + 1) * cfg.G)
    a, _ = osc.window_scores(f64(q[l:l + 1, heads]), f64(k[l:l + 1, g:g + 1]))
    return osc.pool1d(a[0, 0], cfg.pool, cfg.pool_k)


def test_tiny_workload_end_to_end():
    dev = require_gpu()
    cfg = wl.CONFIGS["tiny"]
    inp = wl.tiny_inputs(cfg, dev)
    scores, kept, mask, dk, dv = _token_path(dev, cfg, inp)
    q, k, v = inp["q"], inp["k"], inp["v"]
    a, _ = osc.window_scores(f64(q), f64(k))
    assert_scores_close(f64(scores), a.reshape(cfg.U, cfg.N))
    pooled = osc.pool1d(a, cfg.pool, cfg.pool_k).reshape(cfg.U, cfg.N)
    kn, vn, kept_h = f64(k).reshape(cfg.U, cfg.N, cfg.D), f64(v).reshape(cfg.U, cfg.N, cfg.D), kept.cpu().numpy()
    for u in range(cfg.U):
        s32 = numerics.round_to_f32(pooled[u])
        verdict = check_selection(kept_h[u], s32, cfg.k, cfg.n_sink, cfg.n_recent, what="unit %d" % u)
        ok, om_ = osel_topk(s32, cfg)
        if verdict == "exact":
            np.testing.assert_array_equal(mask[u].cpu().numpy().astype(bool), om_)
            gk, gv = om.gather_view(kn[u], vn[u], ok, 1)
            np.testing.assert_array_equal(f64(dk[u]), gk)
            np.testing.assert_array_equal(f64(dv[u]), gv)


def osel_topk(s32, cfg):
    from oracle import select as osel
    return osel.select_topk(s32, cfg.k, cfg.n_sink, cfg.n_recent)


@pytest.mark.timeout(900)
def test_snapkv_workload_full_size():
    """The full 36 x 8 x 32768 x 128 bf16 workload in the launch sequence
    the benchmark times: the LSE pass, the score pass with that LSE, select
    with max-pool 7 in its own workgroup's registers, and the gather.  Every
    one of the 288 units is checked against the oracle: the LSE and the
    scores element by element, the kept indices bit for bit (or under the
    near-tie rule), and on every bit-exact unit the gathered K and V."""
    dev = require_gpu()
    cfg = wl.CONFIGS["snapkv"]
    inp = wl.snapkv_inputs(cfg, dev)
    q, k, v = inp["q"], inp["k"], inp["v"]
    U, N, D = cfg.U, cfg.N, cfg.D
    lse = torch.empty((cfg.L, cfg.Hq, cfg.W), dtype=torch.float32, device=dev)
    scores = torch.empty((U, N), dtype=torch.float32, device=dev)
    kept = torch.empty((U, cfg.k), dtype=torch.int32, device=dev)
    dk = torch.empty((U, cfg.k, D), dtype=k.dtype, device=dev)
    dv = torch.empty_like(dk)
    kv.score_window(q, k, None, lse_out=lse)
    kv.score_window(q, k, scores, lse_in=lse)
    kv.select(scores, kept, k_total=cfg.k, n_sink=cfg.n_sink, n_recent=cfg.n_recent, pool=cfg.pool,
              pool_k=cfg.pool_k)
    kv.gather_rerope(k.view(U, N, D), v.view(U, N, D), kept, dk, dv, bt=1, D=D, src_rows=N, src_unit_stride=N * D)
    torch.cuda.synchronize()
    kept_h, lse_h = kept.cpu().numpy(), f64(lse)
    cond = Conditioning("snapkv")
    for u in range(U):
        l, g = divmod(u, cfg.Hkv)
        heads = slice(g * cfg.G, (g + 1) * cfg.G)
        a, ol = osc.window_scores(f64(q[l:l + 1, heads]), f64(k[l:l + 1, g:g + 1]))
        assert_scores_close(lse_h[l, heads].reshape(1, -1), ol.reshape(1, -1), "lse of unit %d" % u)
        assert_scores_close(f64(scores[u])[None], a[0, 0][None], "unit %d" % u)
        s32 = numerics.round_to_f32(osc.pool1d(a[0, 0], cfg.pool, cfg.pool_k))
        verdict = check_selection(kept_h[u], s32, cfg.k, cfg.n_sink, cfg.n_recent, what="unit %d" % u)
        cond.add(verdict, boundary_gap(s32, cfg.k, cfg.n_sink, cfg.n_recent))
        if verdict == "exact":
            gk, gv = om.gather_view(f64(k[l, g]), f64(v[l, g]), kept_h[u], 1)
            np.testing.assert_array_equal(f64(dk[u]), gk)
            np.testing.assert_array_equal(f64(dv[u]), gv)
            cond.materialised += 1
    print(cond.report(), flush=True)
    assert cond.exact >= 0.8 * U and cond.materialised == cond.exact
    assert np.all(kept_h[:, : cfg.n_sink] == np.arange(cfg.n_sink))
    assert np.all(kept_h[:, -cfg.n_recent:] == np.arange(N - cfg.n_recent, N))
    assert np.all(np.diff(kept_h, axis=1) > 0)
