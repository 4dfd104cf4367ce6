"""GPU parity of the session-memory path: kvsel_memory_update, kvsel_score
(memory mode over a paged pool), global kvsel_select with dead positions,
and kvsel_redirect with the dead-slot sentinel."""
import math

import numpy as np
import pytest
import torch

from oracle import materialise as om
from oracle import numerics
from oracle import score as osc
from oracle import select as osel
from parity import Conditioning, boundary_gap, assert_scores_close, check_selection, f64, require_gpu

import selection_score_amd as kv
from selection_score_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _small_pool(dev, L=2, Hq=8, Hkv=2, D=128, N=1000, ps=16, seed=0, dtype=torch.bfloat16):
    g = torch.Generator(device=dev).manual_seed(seed)
    n_pages = (N + ps - 1) // ps
    P = n_pages + 3
    k_pool = torch.randn((L, P, ps, Hkv, D), generator=g, device=dev).to(dtype)
    perm = torch.randperm(P, generator=g, device=dev)[:n_pages].to(torch.int32)
    return k_pool, perm, n_pages


@pytest.mark.parametrize("dtype,W", [(torch.bfloat16, 64), (torch.float32, 5)])
def test_memory_update_matches_oracle(dtype, W):
    dev = require_gpu()
    g = torch.Generator(device=dev).manual_seed(W)
    L, Hq, D = 3, 8, 128
    m = torch.zeros((L, Hq, D), dtype=torch.float32, device=dev)
    mo = np.zeros((L, Hq, D))
    for t in range(4):
        qt = (torch.randn((L, Hq, W, D), generator=g, device=dev) + t).to(dtype)
        kv.memory_update(qt, m, decay=0.9)
        mo = osc.memory_update(mo, f64(qt), decay=0.9)
    torch.cuda.synchronize()
    np.testing.assert_allclose(f64(m), mo, rtol=0, atol=2e-6)
    np.testing.assert_allclose(np.linalg.norm(f64(m), axis=-1), 1.0, atol=1e-5)


@pytest.mark.parametrize("reduce,Hq,Hkv,D,ps,dtype", [
    ("global", 8, 2, 128, 16, torch.bfloat16),      # matrix cores, GQA 4, one 16-head block
    ("per_unit", 8, 2, 128, 16, torch.bfloat16),
    ("global", 32, 4, 128, 16, torch.bfloat16),     # matrix cores, GQA 8, two head blocks
    ("per_unit", 16, 1, 128, 16, torch.bfloat16),   # matrix cores, GQA 16
    ("global", 8, 4, 128, 16, torch.bfloat16),      # GQA 2: vector ALUs
    ("global", 8, 2, 64, 8, torch.float16),         # fp16, D 64, 8-token pages: vector ALUs
    ("per_unit", 8, 2, 128, 64, torch.bfloat16),    # 64-token pages: vector ALUs, 68 KiB of LDS staging
    ("global", 4, 1, 128, 32, torch.float16),       # 32-token pages, one KV head
])
def test_memory_scores_match_oracle(reduce, Hq, Hkv, D, ps, dtype):
    dev = require_gpu()
    L, N = 2, 1000
    k_pool, perm, n_pages = _small_pool(dev, L, Hq, Hkv, D, N, ps, dtype=dtype)
    rng = np.random.default_rng(1)
    mo = osc.memory_update(np.zeros((L, Hq, D)), rng.standard_normal((L, Hq, 3, D)))
    m32 = numerics.round_to_f32(mo)
    dead = 10 ** 6
    j = np.arange(N)
    slot_map = perm.cpu().numpy().astype(np.int64)[j // ps] * ps + j % ps
    slot_map[rng.choice(N, 40, replace=False)] = dead
    sm = torch.from_numpy(slot_map.astype(np.int32)).to(dev)
    out = torch.empty((N,) if reduce == "global" else (L * Hkv, N), dtype=torch.float32, device=dev)
    kv.score_memory(torch.from_numpy(m32).to(dev), k_pool, perm, N, out, page_size=ps, slot_map=sm,
                    dead_slot=dead, n_sink=4, n_recent=9, reduce=reduce)
    torch.cuda.synchronize()
    want = osc.memory_scores(m32.astype(np.float64), f64(k_pool), perm.cpu().numpy(), ps, N,
                             slot_map=slot_map, dead_slot=dead, n_sink=4, n_recent=9, reduce=reduce)
    assert_scores_close(f64(out).reshape(-1, N), want.reshape(-1, N))
    if reduce == "global":
        assert abs(float(out.sum()) - L * Hq) < 1e-3 * L * Hq
    # a workspace one layer of logit scratch short: two passes, the same bits
    full = kv.score_memory(torch.from_numpy(m32).to(dev), k_pool, perm, N, out, page_size=ps, slot_map=sm,
                           dead_slot=dead, n_sink=4, n_recent=9, reduce=reduce)
    layer = (Hq * N * 4 + 255) // 256 * 256
    out2 = torch.full_like(out, -1.0)
    kv.score_memory(torch.from_numpy(m32).to(dev), k_pool, perm, N, out2, page_size=ps, slot_map=sm,
                    dead_slot=dead, n_sink=4, n_recent=9, reduce=reduce, workspace=full[: full.numel() - layer])
    torch.cuda.synchronize()
    assert torch.equal(out2, out)
    with pytest.raises(kv.KvselError) as e:
        kv.score_memory(torch.from_numpy(m32).to(dev), k_pool, perm, N, out2, page_size=ps, slot_map=sm,
                        dead_slot=dead, n_sink=4, n_recent=9, reduce=reduce,
                        workspace=full[: full.numel() - 2 * layer + 256])
    assert e.value.status == 4


def test_redirect_and_sentinel():
    dev = require_gpu()
    rng = np.random.default_rng(2)
    L, Hkv, D, ps, P = 3, 2, 128, 16, 9
    N, dead = 100, (P - 1) * ps
    slot_map = rng.permutation((P - 1) * ps)[:N].astype(np.int64)
    slot_map[[5, 6]] = dead
    keep = (rng.random(N) > 0.5).astype(np.uint8)
    keep[5] = 1
    for dtype, bits in [(torch.bfloat16, 0xC61C), (torch.float16, 0xF0E2)]:
        k_pool = torch.randn((L, P * ps, Hkv, D), device=dev).to(dtype)
        v_pool = torch.randn_like(k_pool)
        sm = torch.from_numpy(slot_map.astype(np.int32)).to(dev)
        kv.redirect(sm, torch.from_numpy(keep).to(dev), dead, k_pool=k_pool, v_pool=v_pool)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(sm.cpu().numpy(), om.redirect(slot_map, keep, dead))
        kb = k_pool[:, dead].contiguous().view(torch.int16).cpu().numpy().astype(np.uint16)
        assert np.all(kb == bits)
        assert torch.all(v_pool[:, dead] == 0)
        kbo, _ = om.sentinel_rows("bf16" if dtype == torch.bfloat16 else "f16", D)
        np.testing.assert_array_equal(f64(k_pool[0, dead, 0]), kbo)
        # other slots untouched
        assert torch.isfinite(k_pool[:, :dead].float()).all()

    # the kept set given as kvsel_select's ascending list with its -1 tail
    # (and a position past N, which never matches) instead of the mask
    kept = np.flatnonzero(keep).astype(np.int32)
    for tail in (0, 7):
        lst = np.concatenate([kept, [N + 3] if tail else [], np.full(tail, -1)]).astype(np.int32)
        sm = torch.from_numpy(slot_map.astype(np.int32)).to(dev)
        kv.redirect(sm, None, dead, kept_idx=torch.from_numpy(lst).to(dev))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(sm.cpu().numpy(), om.redirect(slot_map, keep, dead))
    # an empty list drops everything
    sm = torch.from_numpy(slot_map.astype(np.int32)).to(dev)
    kv.redirect(sm, None, dead, kept_idx=torch.empty(0, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert np.all(sm.cpu().numpy() == dead)


def test_intentkv_workload_full_size():
    """The session-memory workload at full size: 8 turns of memory updates,
    rule scores over the 36 x 65536 paged pool, global top-8192 with
    4 sink + 64 recent, redirect of the rest to the dead slot."""
    dev = require_gpu()
    cfg = wl.CONFIGS["intentkv"]
    inp = wl.intentkv_inputs(cfg, dev)
    L, Hq, D, N, ps = cfg.L, cfg.Hq, cfg.D, cfg.N, cfg.page_size
    # memory update: GPU against the oracle, turn by turn
    m = torch.zeros((L, Hq, D), dtype=torch.float32, device=dev)
    mo = np.zeros((L, Hq, D))
    for qt in inp["turns"]:
        kv.memory_update(qt, m, decay=cfg.decay)
        mo = osc.memory_update(mo, f64(qt), decay=cfg.decay)
    torch.cuda.synchronize()
    np.testing.assert_allclose(f64(m), mo, rtol=0, atol=2e-6)
    # rule scores from the oracle's memory (float32), every position checked
    m32 = numerics.round_to_f32(mo)
    k_pool, page_table, slot_map, dead = inp["k_pool"], inp["page_table"], inp["slot_map"], inp["dead_slot"]
    rule = torch.empty(N, dtype=torch.float32, device=dev)
    kv.score_memory(torch.from_numpy(m32).to(dev), k_pool, page_table, N, rule, page_size=ps,
                    slot_map=slot_map, dead_slot=dead, n_sink=cfg.n_sink, n_recent=cfg.n_recent)
    kept = torch.empty((1, cfg.k), dtype=torch.int32, device=dev)
    mask = torch.empty((1, N), dtype=torch.uint8, device=dev)
    kv.select(rule[None], kept, k_total=cfg.k, n_sink=cfg.n_sink, n_recent=cfg.n_recent, keep_mask=mask,
              slot_map=slot_map, dead_slot=dead)
    sm_new = slot_map.clone()
    kv_pool_flat = k_pool.view(L, -1, cfg.Hkv, D)
    v_pool_flat = inp["v_pool"].view(L, -1, cfg.Hkv, D)
    kv.redirect(sm_new, mask[0], dead, k_pool=kv_pool_flat, v_pool=v_pool_flat)
    torch.cuda.synchronize()
    pt_h, sm_h = page_table.cpu().numpy(), slot_map.cpu().numpy().astype(np.int64)
    want = np.zeros(N)
    pool64 = None
    for l in range(L):                     # one layer at a time keeps host memory bounded
        pool64 = f64(k_pool[l:l + 1])
        want += osc.memory_scores(m32[l:l + 1].astype(np.float64), pool64, pt_h, ps, N, slot_map=sm_h,
                                  dead_slot=dead, n_sink=cfg.n_sink, n_recent=cfg.n_recent)
    del pool64
    got = f64(rule)
    assert_scores_close(got[None], want[None])
    assert abs(got.sum() - L * Hq) < 1e-3 * L * Hq
    s32 = numerics.round_to_f32(want)
    verdict = check_selection(kept.cpu().numpy()[0], s32, cfg.k, cfg.n_sink, cfg.n_recent,
                              alive=sm_h != dead)
    cond = Conditioning("intentkv")
    cond.add(verdict, boundary_gap(s32, cfg.k, cfg.n_sink, cfg.n_recent, sm_h != dead))
    if verdict == "exact":
        _, om_mask = osel.select_topk(s32, cfg.k, cfg.n_sink, cfg.n_recent, sm_h != dead)
        np.testing.assert_array_equal(sm_new.cpu().numpy(), om.redirect(sm_h, om_mask, dead))
        cond.materialised += 1
    print(cond.report(), flush=True)
    # survivors unmoved, the rest on the dead slot, sentinel rows written
    new_h = sm_new.cpu().numpy()
    keep_h = mask.cpu().numpy()[0].astype(bool)
    np.testing.assert_array_equal(new_h[keep_h], sm_h[keep_h])
    assert np.all(new_h[~keep_h] == dead) and int(keep_h.sum()) == cfg.k
    kb = kv_pool_flat[:, dead].contiguous().view(torch.int16).cpu().numpy().astype(np.uint16)
    assert np.all(kb == 0xC61C) and torch.all(v_pool_flat[:, dead] == 0)
    # decode attention through the redirected map equals the hard mask for a
    # query whose entries sum well above the sentinel margin (layer 0, head 0)
    layer = 0
    kl = f64(kv_pool_flat[layer, :, 0])
    vl = f64(v_pool_flat[layer, :, 0])
    q = np.abs(np.random.default_rng(3).standard_normal(D)) * 0.2
    assert q.sum() * 9984 / math.sqrt(D) > 800
    o_dead = om.decode_attention_slots(q, kl, vl, new_h)
    o_hard = om.decode_attention_hard(q, kl, vl, sm_h, keep_h)
    np.testing.assert_array_equal(o_dead, o_hard)
