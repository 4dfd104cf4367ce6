"""GPU parity of kvsel_gather_rerope (fresh and incremental) against the oracle."""
import numpy as np
import pytest
import torch

from oracle import materialise as om
from oracle import numerics
from oracle.rope import rope_rotate
from parity import assert_rope_close, f64, require_gpu

import selection_score_amd as kv

pytestmark = pytest.mark.gpu


def _idx(rng, U, nb, k):
    return np.stack([np.sort(rng.choice(nb, k, replace=False)) for _ in range(U)]).astype(np.int32)


@pytest.mark.parametrize("dtype,D,bt", [(torch.bfloat16, 128, 1), (torch.float32, 64, 1),
                                        (torch.float16, 128, 32), (torch.bfloat16, 64, 4)])
def test_gather_plain_is_bitwise(dtype, D, bt):
    dev = require_gpu()
    rng = np.random.default_rng(D + bt)
    U, nb, k = 5, 777, 131
    g = torch.Generator(device=dev).manual_seed(5)
    src_k = torch.randn((U, nb * bt, D), generator=g, device=dev).to(dtype)
    src_v = torch.randn((U, nb * bt, D), generator=g, device=dev).to(dtype)
    idx = _idx(rng, U, nb, k)
    it = torch.from_numpy(idx).to(dev)
    dk = torch.empty((U, k * bt, D), dtype=dtype, device=dev)
    dv = torch.empty_like(dk)
    kv.gather_rerope(src_k, src_v, it, dk, dv, bt=bt, D=D, src_rows=nb * bt,
                     src_unit_stride=nb * bt * D)
    torch.cuda.synchronize()
    sk, sv = f64(src_k), f64(src_v)
    for u in range(U):
        ok, ov = om.gather_view(sk[u], sv[u], idx[u], bt)
        np.testing.assert_array_equal(f64(dk[u]), ok)
        np.testing.assert_array_equal(f64(dv[u]), ov)


@pytest.mark.parametrize("bt,rope,style,pos0", [(32, "raw", "half", 0), (32, "raw", "interleaved", 100),
                                                (32, "delta", "half", 0), (1, "raw", "half", 12345),
                                                (8, "delta", "interleaved", 7)])
def test_gather_rerope_matches_oracle(bt, rope, style, pos0):
    dev = require_gpu()
    rng = np.random.default_rng(bt * 3 + len(rope))
    U, nb, k, D = 6, 3000, 257, 128
    g = torch.Generator(device=dev).manual_seed(6)
    src_k = torch.randn((U, nb * bt, D), generator=g, device=dev).to(torch.bfloat16)
    src_v = torch.randn((U, nb * bt, D), generator=g, device=dev).to(torch.bfloat16)
    idx = _idx(rng, U, nb - 1, k - 1)
    idx = np.concatenate([idx, np.full((U, 1), nb - 1, np.int32)], axis=1)   # largest angles
    it = torch.from_numpy(idx).to(dev)
    dk = torch.empty((U, k * bt, D), dtype=torch.bfloat16, device=dev)
    dv = torch.empty_like(dk)
    kv.gather_rerope(src_k, src_v, it, dk, dv, bt=bt, D=D, src_rows=nb * bt, src_unit_stride=nb * bt * D,
                     rope=rope, theta=1e6, pos0=pos0, style=style)
    torch.cuda.synchronize()
    sk, sv = f64(src_k), f64(src_v)
    for u in range(U):
        ok, ov = om.gather_view(sk[u], sv[u], idx[u], bt, rope=rope, theta=1e6, pos0=pos0, style=style)
        assert_rope_close(f64(dk[u]), ok, "unit %d" % u, style=style)
        np.testing.assert_array_equal(f64(dv[u]), ov)


@pytest.mark.parametrize("dtype,D,rope,style", [(torch.float16, 64, "raw", "interleaved"),
                                               (torch.float32, 128, "delta", "half"),
                                               (torch.float32, 64, "raw", "half"),
                                               (torch.float16, 128, "delta", "interleaved")])
def test_gather_blocks_dtypes(dtype, D, rope, style):
    """The block gather (K rotation and V copy of an entry in separate
    wavefronts) for fp16 and fp32 K/V and head dims 64 and 128."""
    dev = require_gpu()
    rnd = {torch.float16: numerics.round_to_f16, torch.float32: numerics.round_to_f32}[dtype]
    rng = np.random.default_rng(D + len(rope) + len(style))
    U, nb, k, bt = 4, 800, 97, 16
    sk = rnd(rng.standard_normal((U, nb * bt, D)))
    sv = rnd(rng.standard_normal((U, nb * bt, D)))
    idx = _idx(rng, U, nb, k)
    t = lambda x: torch.from_numpy(x.astype(np.float32)).to(dtype).to(dev)
    dk = torch.empty((U, k * bt, D), dtype=dtype, device=dev)
    dv = torch.empty_like(dk)
    kv.gather_rerope(t(sk), t(sv), torch.from_numpy(idx).to(dev), dk, dv, bt=bt, D=D, src_rows=nb * bt,
                     src_unit_stride=nb * bt * D, rope=rope, theta=1e6, pos0=9, style=style)
    torch.cuda.synchronize()
    for u in range(U):
        ok, ov = om.gather_view(sk[u], sv[u], idx[u], bt, rope=rope, theta=1e6, pos0=9, style=style, out_round=rnd)
        assert_rope_close(f64(dk[u]), ok, "unit %d" % u, style=style)
        np.testing.assert_array_equal(f64(dv[u]), ov)


def test_gather_zero_rotation_is_bitwise():
    # DELTA with every entry at its own position: R(0) must pass K through untouched
    dev = require_gpu()
    U, nb, D, bt = 2, 64, 128, 32
    g = torch.Generator(device=dev).manual_seed(8)
    src_k = torch.randn((U, nb * bt, D), generator=g, device=dev).to(torch.bfloat16)
    idx = torch.arange(nb, dtype=torch.int32, device=dev).repeat(U, 1).contiguous()
    dk = torch.empty((U, nb * bt, D), dtype=torch.bfloat16, device=dev)
    dv = torch.empty_like(dk)
    kv.gather_rerope(src_k, src_k, idx, dk, dv, bt=bt, D=D, src_rows=nb * bt, src_unit_stride=nb * bt * D,
                     rope="delta", theta=1e6)
    torch.cuda.synchronize()
    assert torch.equal(dk.view(torch.int16), src_k.view(torch.int16))


def test_gather_aliased_sources_and_partial_counts():
    # units share physical source buffers through per-unit offsets; n_idx
    # limits each unit's entries (the rest of dst stays untouched)
    dev = require_gpu()
    rng = np.random.default_rng(9)
    n_buf, U, nb, k, D, bt = 2, 6, 500, 40, 128, 32
    g = torch.Generator(device=dev).manual_seed(9)
    src_k = torch.randn((n_buf, nb * bt, D), generator=g, device=dev).to(torch.bfloat16)
    src_v = torch.randn((n_buf, nb * bt, D), generator=g, device=dev).to(torch.bfloat16)
    offs = torch.tensor([(u % n_buf) * nb * bt * D for u in range(U)], dtype=torch.int64, device=dev)
    idx = _idx(rng, U, nb, k)
    n_idx = np.array([k, 0, 17, k, 1, 39], np.int32)
    dk = torch.full((U, k * bt, D), 3.0, dtype=torch.bfloat16, device=dev)
    dv = torch.full_like(dk, 5.0)
    kv.gather_rerope(src_k, src_v, torch.from_numpy(idx).to(dev), dk, dv, bt=bt, D=D, src_rows=nb * bt,
                     src_offsets=offs, n_idx=torch.from_numpy(n_idx).to(dev), rope="raw", theta=1e6)
    torch.cuda.synchronize()
    sk, sv = f64(src_k), f64(src_v)
    for u in range(U):
        m = int(n_idx[u])
        ok, ov = om.gather_view(sk[u % n_buf], sv[u % n_buf], idx[u, :m], bt, rope="raw", theta=1e6)
        got_k, got_v = f64(dk[u]), f64(dv[u])
        if m:
            assert_rope_close(got_k[: m * bt], ok)
            np.testing.assert_array_equal(got_v[: m * bt], ov)
        assert np.all(got_k[m * bt:] == 3.0) and np.all(got_v[m * bt:] == 5.0)


_ROUND = {torch.bfloat16: numerics.round_to_bf16, torch.float16: numerics.round_to_f16,
          torch.float32: numerics.round_to_f32}


@pytest.mark.parametrize("dtype,D,style,hits,pos0", [(torch.float16, 64, "interleaved", "raw", 0),
                                                     (torch.float32, 128, "half", "delta", 300),
                                                     (torch.bfloat16, 64, "interleaved", "delta", 17),
                                                     (torch.float32, 64, "half", "raw", 5)])
def test_incremental_view_dtypes_and_styles(dtype, D, style, hits, pos0):
    """The incremental view (K and V of an entry moved by separate
    wavefronts) for fp16/fp32/bf16 pools, head dims 64 and 128, both
    rotation styles, a non-zero base position and both hit modes: page
    table and V bit for bit, K within the re-RoPE bar (bf16's, which holds
    the narrower formats too)."""
    dev = require_gpu()
    rnd = _ROUND[dtype]
    rng = np.random.default_rng(D + len(style) + pos0)
    U, nb, k, bt, spare = 3, 600, 64, 16, 6
    P = k + spare
    raw_k = rnd(rng.standard_normal((U, nb * bt, D)))
    raw_v = rnd(rng.standard_normal((U, nb * bt, D)))
    new_idx, prev_idx, prev_page = [], [], []
    for u in range(U):
        new = np.sort(rng.choice(nb, k, replace=False))
        outside = np.setdiff1d(np.arange(nb), new)
        prev = np.sort(np.concatenate([rng.choice(new, k // 2, replace=False),
                                       rng.choice(outside, k - k // 2, replace=False)]))
        new_idx.append(new)
        prev_idx.append(prev)
        prev_page.append(rng.permutation(P)[:k])
    new_idx, prev_idx, prev_page = (np.stack(x).astype(np.int32) for x in (new_idx, prev_idx, prev_page))
    o = np.arange(bt)
    pool_k = rnd(rng.standard_normal((U, P, bt, D)))
    pool_v = rnd(rng.standard_normal((U, P, bt, D)))
    for u in range(U):
        for i, b in enumerate(prev_idx[u]):
            pool_k[u, prev_page[u, i]] = rnd(rope_rotate(raw_k[u, b * bt:(b + 1) * bt], pos0 + i * bt + o, 1e6,
                                                         style=style))
            pool_v[u, prev_page[u, i]] = raw_v[u, b * bt:(b + 1) * bt]
    t = lambda x: torch.from_numpy(x.astype(np.float32)).to(dtype).to(dev)
    rk_t, rv_t, pk, pv = t(raw_k), t(raw_v), t(pool_k), t(pool_v)
    pt = torch.full((U, k), -5, dtype=torch.int32, device=dev)
    nm = torch.zeros(U, dtype=torch.int32, device=dev)
    kv.gather_incremental(rk_t, rv_t, torch.from_numpy(new_idx).to(dev), torch.from_numpy(prev_idx).to(dev),
                          torch.from_numpy(prev_page).to(dev), pk, pv, pt, nm, bt=bt, D=D, src_rows=nb * bt,
                          src_unit_stride=nb * bt * D, rope="raw", theta=1e6, pos0=pos0, style=style,
                          hit_raw=hits == "raw")
    torch.cuda.synchronize()
    gk, gv, gpt, gnm = f64(pk), f64(pv), pt.cpu().numpy(), nm.cpu().numpy()
    for u in range(U):
        ok, ov, opt, onm = om.incremental_view(prev_idx[u], prev_page[u], new_idx[u], pool_k[u], pool_v[u],
                                               raw_k[u].reshape(nb, bt, D), raw_v[u].reshape(nb, bt, D), bt,
                                               theta=1e6, pos0=pos0, style=style, out_round=rnd, hits=hits)
        assert gnm[u] == onm
        np.testing.assert_array_equal(gpt[u], opt)
        np.testing.assert_array_equal(gv[u], ov)
        assert_rope_close(gk[u], ok, "unit %d" % u, style=style)


@pytest.mark.parametrize("overlap,staged,hits", [(0.5, False, "delta"), (1.0, False, "delta"), (0.0, False, "delta"),
                                                 (0.5, True, "delta"), (0.0, True, "delta"), (0.5, False, "raw"),
                                                 (1.0, True, "raw")])
def test_incremental_view_matches_oracle(overlap, staged, hits):
    """The incremental view against the oracle's, with the misses read from
    the raw source by block id or from packed staging buffers (the i-th miss
    of a unit, in ascending block order, at entry i; no raw source given
    unless moved hits are re-rotated from it), and moved hits rotated in
    place or re-rotated from raw K."""
    dev = require_gpu()
    rng = np.random.default_rng(int(overlap * 10) + 11)
    U, nb, k, D, bt, spare = 4, 2000, 96, 128, 32, 10
    P = k + spare
    g = torch.Generator(device=dev).manual_seed(12)
    raw_k = torch.randn((U, nb * bt, D), generator=g, device=dev).to(torch.bfloat16)
    raw_v = torch.randn((U, nb * bt, D), generator=g, device=dev).to(torch.bfloat16)
    new_idx, prev_idx, prev_page = [], [], []
    for u in range(U):
        new = np.sort(rng.choice(nb, k, replace=False))
        n_keep = int(round(k * overlap))
        outside = np.setdiff1d(np.arange(nb), new)
        prev = np.sort(np.concatenate([rng.choice(new, n_keep, replace=False),
                                       rng.choice(outside, k - n_keep, replace=False)]))
        new_idx.append(new)
        prev_idx.append(prev)
        prev_page.append(rng.permutation(P)[:k])
    new_idx, prev_idx, prev_page = (np.stack(x).astype(np.int32) for x in (new_idx, prev_idx, prev_page))
    # previous view: raw K baked at its old positions (computed by the oracle)
    rk, rv = f64(raw_k), f64(raw_v)
    pool_k = numerics.round_to_bf16(np.random.default_rng(13).standard_normal((U, P, bt, D)))
    pool_v = numerics.round_to_bf16(np.random.default_rng(14).standard_normal((U, P, bt, D)))
    o = np.arange(bt)
    for u in range(U):
        for i, b in enumerate(prev_idx[u]):
            pool_k[u, prev_page[u, i]] = numerics.round_to_bf16(
                rope_rotate(rk[u, b * bt:(b + 1) * bt], i * bt + o, 1e6))
            pool_v[u, prev_page[u, i]] = rv[u, b * bt:(b + 1) * bt]
    pk = torch.from_numpy(pool_k.astype(np.float32)).to(torch.bfloat16).to(dev)
    pv = torch.from_numpy(pool_v.astype(np.float32)).to(torch.bfloat16).to(dev)
    pt = torch.full((U, k), -5, dtype=torch.int32, device=dev)
    nm = torch.zeros(U, dtype=torch.int32, device=dev)
    if staged:
        # the host side of the tiered movement: missed blocks packed in ascending block order
        sk = torch.zeros((U, k, bt, D), dtype=torch.bfloat16, device=dev)
        sv = torch.zeros_like(sk)
        for u in range(U):
            miss = np.setdiff1d(new_idx[u], prev_idx[u])
            rows = torch.from_numpy((miss[:, None] * bt + np.arange(bt)).reshape(-1)).to(dev)
            sk[u, :len(miss)] = raw_k[u][rows].view(len(miss), bt, D)
            sv[u, :len(miss)] = raw_v[u][rows].view(len(miss), bt, D)
        src = (raw_k, raw_v) if hits == "raw" else (None, None)
        kv.gather_incremental(*src, torch.from_numpy(new_idx).to(dev), torch.from_numpy(prev_idx).to(dev),
                              torch.from_numpy(prev_page).to(dev), pk, pv, pt, nm, bt=bt, D=D, rope="raw",
                              theta=1e6, staged_k=sk, staged_v=sv, hit_raw=hits == "raw", src_rows=nb * bt,
                              src_unit_stride=nb * bt * D)
    else:
        kv.gather_incremental(raw_k, raw_v, torch.from_numpy(new_idx).to(dev), torch.from_numpy(prev_idx).to(dev),
                              torch.from_numpy(prev_page).to(dev), pk, pv, pt, nm, bt=bt, D=D,
                              src_rows=nb * bt, src_unit_stride=nb * bt * D, rope="raw", theta=1e6,
                              hit_raw=hits == "raw")
    torch.cuda.synchronize()
    gk, gv, gpt, gnm = f64(pk), f64(pv), pt.cpu().numpy(), nm.cpu().numpy()
    for u in range(U):
        ok, ov, opt, onm = om.incremental_view(prev_idx[u], prev_page[u], new_idx[u], pool_k[u], pool_v[u],
                                               rk[u].reshape(nb, bt, D), rv[u].reshape(nb, bt, D), bt,
                                               theta=1e6, hits=hits)
        assert gnm[u] == onm
        np.testing.assert_array_equal(gpt[u], opt)
        np.testing.assert_array_equal(gv[u], ov)
        assert_rope_close(gk[u], ok, "pool unit %d" % u)


def test_incremental_staging_shorter_than_the_misses():
    """Misses beyond the staging capacity are skipped: their pages keep their
    bytes, every other page is as the oracle builds it."""
    dev = require_gpu()
    rng = np.random.default_rng(21)
    nb, k, D, bt, cap = 300, 40, 128, 32, 7
    raw_k = torch.randn((nb * bt, D), generator=torch.Generator(device=dev).manual_seed(3), device=dev).to(torch.bfloat16)
    raw_v = torch.randn_like(raw_k)
    new = np.sort(rng.choice(nb, k, replace=False))
    prev = np.sort(np.concatenate([new[: k - 10], rng.choice(np.setdiff1d(np.arange(nb), new), 10, replace=False)]))
    page = rng.permutation(k + 3)[:k].astype(np.int32)
    miss = np.setdiff1d(new, prev)
    assert len(miss) == 10 > cap
    pool0 = numerics.round_to_bf16(np.random.default_rng(22).standard_normal((k + 3, bt, D)))
    pk = torch.from_numpy(pool0.astype(np.float32)).to(torch.bfloat16).to(dev)[None].contiguous()
    pv = pk.clone()
    rows = torch.from_numpy((miss[:cap, None] * bt + np.arange(bt)).reshape(-1)).to(dev)
    sk = raw_k[rows].view(1, cap, bt, D).contiguous()
    sv = raw_v[rows].view(1, cap, bt, D).contiguous()
    pt = torch.empty((1, k), dtype=torch.int32, device=dev)
    nm = torch.empty(1, dtype=torch.int32, device=dev)
    t = lambda x: torch.from_numpy(np.asarray(x, np.int32)[None]).to(dev)
    kv.gather_incremental(None, None, t(new), t(prev), t(page), pk, pv, pt, nm, bt=bt, D=D, rope="raw", theta=1e6,
                          staged_k=sk, staged_v=sv)
    torch.cuda.synchronize()
    ok, ov, opt, onm = om.incremental_view(prev, page, new, pool0, pool0, f64(raw_k).reshape(nb, bt, D),
                                           f64(raw_v).reshape(nb, bt, D), bt, theta=1e6)
    assert int(nm[0]) == onm == len(miss)
    gpt = pt.cpu().numpy()[0]
    np.testing.assert_array_equal(gpt, opt)
    skipped = set(gpt[np.isin(new, miss[cap:])].tolist())
    gk, gv = f64(pk[0]), f64(pv[0])
    for pg in range(k + 3):
        if pg in skipped:
            np.testing.assert_array_equal(gk[pg], pool0[pg])
            np.testing.assert_array_equal(gv[pg], pool0[pg])
        else:
            assert_rope_close(gk[pg], ok[pg], "page %d" % pg)
            np.testing.assert_array_equal(gv[pg], ov[pg])
