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


@pytest.mark.parametrize("overlap", [0.5, 1.0, 0.0])
def test_incremental_view_matches_oracle(overlap):
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
    kv.gather_incremental(raw_k, raw_v, torch.from_numpy(new_idx).to(dev), torch.from_numpy(prev_idx).to(dev),
                          torch.from_numpy(prev_page).to(dev), pk, pv, pt, nm, bt=bt, D=D,
                          src_rows=nb * bt, src_unit_stride=nb * bt * D, rope="raw", theta=1e6)
    torch.cuda.synchronize()
    gk, gv, gpt, gnm = f64(pk), f64(pv), pt.cpu().numpy(), nm.cpu().numpy()
    for u in range(U):
        ok, ov, opt, onm = om.incremental_view(prev_idx[u], prev_page[u], new_idx[u], pool_k[u], pool_v[u],
                                               rk[u].reshape(nb, bt, D), rv[u].reshape(nb, bt, D), bt,
                                               theta=1e6)
        assert gnm[u] == onm
        np.testing.assert_array_equal(gpt[u], opt)
        np.testing.assert_array_equal(gv[u], ov)
        assert_rope_close(gk[u], ok, "pool unit %d" % u)
