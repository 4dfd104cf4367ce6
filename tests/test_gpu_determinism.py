"""Repeated calls on the same inputs give bit-identical outputs.

Every reduction of the library runs in a fixed order (chunk partials merged
in chunk order, per-layer sums in layer order, keep-score bucket sums that
are exact whatever the order of their atomic adds), so two runs of a call
must agree bit for bit, not just within a tolerance.
"""
import pytest
import torch

from parity import require_gpu

import selection_score_amd as kv

pytestmark = pytest.mark.gpu


def _same(a, b):
    if a.dtype.is_floating_point:
        a, b = a.view(torch.int32 if a.element_size() == 4 else torch.int16), \
            b.view(torch.int32 if b.element_size() == 4 else torch.int16)
    return torch.equal(a, b)


def _twice(fn):
    outs = []
    for _ in range(2):
        outs.append([t.clone() for t in fn()])
        torch.cuda.synchronize()
    for x, y in zip(*outs):
        assert _same(x, y)


def test_window_scores_and_lse_repeat_bitwise():
    dev = require_gpu()
    g = torch.Generator(device=dev).manual_seed(1)
    L, Hq, Hkv, W, N, D = 2, 8, 2, 64, 5000, 128
    q = torch.randn((L, Hq, W, D), generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn((L, Hkv, N, D), generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty((L * Hkv, N), device=dev)
    lse = torch.empty((L, Hq, W), device=dev)
    print("determinism: window", flush=True)

    def run():
        kv.score_window(q, k, out, lse_out=lse, pool="max", pool_k=7)
        return [out, lse]
    _twice(run)


def test_memory_rule_scores_repeat_bitwise():
    dev = require_gpu()
    g = torch.Generator(device=dev).manual_seed(2)
    L, Hq, Hkv, D, ps, N = 2, 8, 2, 128, 16, 3000
    pages = (N + ps - 1) // ps
    m = torch.randn((L, Hq, D), generator=g, device=dev)
    pool = torch.randn((L, pages + 3, ps, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
    pt = torch.randperm(pages + 3, generator=g, device=dev)[:pages].to(torch.int32)
    out = torch.empty(N, device=dev)
    print("determinism: memory", flush=True)

    def run():
        kv.score_memory(m, pool, pt, N, out, page_size=ps, n_sink=4, n_recent=64)
        return [out]
    _twice(run)


def test_block_scores_select_and_gather_repeat_bitwise():
    dev = require_gpu()
    g = torch.Generator(device=dev).manual_seed(3)
    S, L, Hq, Hkv, Wq, D, NB, bt, k = 2, 2, 8, 2, 16, 128, 5000, 32, 300
    q = torch.randn((S, L, Hq, Wq, D), generator=g, device=dev).to(torch.bfloat16)
    mu = (torch.randn((L, Hkv, NB, D), generator=g, device=dev) * 0.2).to(torch.float16)
    scores = torch.empty((S, L * Hkv, NB), device=dev)
    U = S * L * Hkv
    kept = torch.empty((U, k), dtype=torch.int32, device=dev)
    raw = torch.randn((L * Hkv, NB * bt, D), generator=g, device=dev).to(torch.bfloat16)
    dk = torch.empty((L * Hkv, k * bt, D), dtype=torch.bfloat16, device=dev)
    dv = torch.empty_like(dk)
    print("determinism: block, select, gather", flush=True)

    def run():
        kv.score_block(q, mu, scores, n_kv_heads=Hkv)
        kv.select(scores.view(U, NB), kept, k_total=k, n_sink=1, n_recent=4)
        kv.gather_rerope(raw, raw, kept[: L * Hkv], dk, dv, bt=bt, D=D, src_rows=NB * bt,
                         src_unit_stride=NB * bt * D, rope="raw", theta=1e6)
        return [scores, kept, dk, dv]
    _twice(run)


def test_decode_state_and_keep_scores_repeat_bitwise():
    dev = require_gpu()
    g = torch.Generator(device=dev).manual_seed(4)
    L, R, Hq, Hkv, D, bs, N = 2, 3, 32, 8, 128, 16, 700
    Y = (N + bs - 1) // bs
    P = R * Y + 2
    q = torch.randn((L, R, Hq, D), generator=g, device=dev).to(torch.bfloat16)
    pool = torch.randn((L, P, bs, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
    bt = torch.randperm(P, generator=g, device=dev)[: R * Y].view(R, Y).to(torch.int32)
    lse = torch.randn((L, R, Hq), generator=g, device=dev) + 8.0
    n_ctx = torch.tensor([700, 513, 64], dtype=torch.int32, device=dev)
    n_seen = torch.tensor([0, 3, 1], dtype=torch.int32, device=dev)
    state0 = torch.rand((L, R, Hkv, N), generator=g, device=dev) * 1e-3
    state0[:, 1, :, 513:] = 0.0
    state0[:, 2, :, 64:] = 0.0
    ks0 = torch.rand((R, N), generator=g, device=dev)
    state = torch.empty_like(state0)
    ks = torch.empty_like(ks0)
    attn = torch.empty((R, N), device=dev)
    hit = torch.empty((R, N), dtype=torch.uint8, device=dev)
    print("determinism: decode, keep score", flush=True)

    def run():
        state.copy_(state0)
        ks.copy_(ks0)
        kv.decode_score(q, lse, pool, bt, n_ctx, n_seen, state)
        kv.keep_score(state, ks, n_ctx, lam=0.5, top_p=0.9, attn_score=attn, hit=hit)
        return [state, ks, attn, hit]
    _twice(run)
