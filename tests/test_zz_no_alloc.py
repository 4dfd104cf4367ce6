"""kvsel_select_noalloc (the select entry point whose scratch is the library's
fixed per-device array) against kvsel_select with a caller workspace: the
same selections bit for bit, on two calls in a row where the second is
smaller, plus the size limit and a tiled call.  Runs last: it shares the
device array with nothing else, and a failure here hides no other test."""
import numpy as np
import pytest
import torch

from parity import require_gpu

import selection_score_amd as kv
from selection_score_amd import _abi

pytestmark = pytest.mark.gpu


def _scores(dev, U, n, seed):
    g = torch.Generator(device=dev).manual_seed(seed)
    s = torch.randn((U, n), generator=g, device=dev)
    s[:, ::97] = 0.5                       # exact ties across the row
    return s


def _both(dev, s, **kw):
    U = s.shape[0]
    k = kw["k_total"]
    n_total = kw.get("n_total", s.shape[1])
    out = []
    for fn in (kv.select, kv.select_noalloc):
        kept = torch.full((U, k), -7, dtype=torch.int32, device=dev)
        mask = torch.full((U, n_total), 9, dtype=torch.uint8, device=dev)
        nk = torch.full((U,), -7, dtype=torch.int32, device=dev)
        fn(s, kept, keep_mask=mask, n_kept=nk, **kw)
        out.append((kept, mask, nk))
    torch.cuda.synchronize()
    return out


def _same(a, b):
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_noalloc_select_equals_workspace_select_on_consecutive_calls():
    dev = require_gpu()
    # first call: 288 units x 32768 columns, avg-pool 7 (the two-launch path,
    # about 40 MB of scratch); second call: a smaller, ragged, avg-pooled one
    # with dead slots, which reuses the front of the same array
    big = _scores(dev, 288, 32768, 1)
    ref, got = _both(dev, big, k_total=8192, n_sink=4, n_recent=256, pool="avg", pool_k=7)
    _same(ref, got)
    assert torch.all(got[2] == 8192)
    small = _scores(dev, 37, 5003, 2)
    dead = torch.zeros(5003, dtype=torch.int32, device=dev)
    dead[::11] = 99
    ref, got = _both(dev, small, k_total=700, n_sink=3, n_recent=40, pool="avg", pool_k=5,
                     slot_map=dead, dead_slot=99)
    _same(ref, got)
    kept = got[0].cpu().numpy()
    assert np.all(kept[:, :700][kept[:, :700] >= 0] % 11 != 0)
    # the first shape again after the smaller one: no stale scratch
    ref, got = _both(dev, big, k_total=8192, n_sink=4, n_recent=256, pool="avg", pool_k=7)
    _same(ref, got)


def test_noalloc_select_without_scratch_use_and_tiled():
    dev = require_gpu()
    # unpooled or max-pooled over a short window, many units: the
    # single-launch path reads no scratch at all
    s = _scores(dev, 512, 32768, 3)
    ref, got = _both(dev, s, k_total=2048, n_sink=1, n_recent=4)
    _same(ref, got)
    ref, got = _both(dev, s[:288], k_total=8192, n_sink=4, n_recent=256, pool="max", pool_k=7)
    _same(ref, got)
    # tiled with running candidates: no scratch either
    U, n_total, tile, k = 9, 100000, 30000, 1024
    full = _scores(dev, U, n_total, 4)
    res = []
    for fn in (kv.select, kv.select_noalloc):
        cs = torch.empty((U, k), device=dev)
        ci = torch.empty((U, k), dtype=torch.int32, device=dev)
        cc = torch.zeros(U, dtype=torch.int32, device=dev)
        kept = torch.empty((U, k), dtype=torch.int32, device=dev)
        for b in range(0, n_total, tile):
            m = min(tile, n_total - b)
            fn(full[:, b:b + m], kept, k_total=k, n_sink=4, n_recent=16, n_total=n_total, base=b,
               cand_score=cs, cand_idx=ci, cand_count=cc, finalize=b + m == n_total)
        res.append(kept)
    torch.cuda.synchronize()
    assert torch.equal(res[0], res[1])


def test_noalloc_select_long_rows_of_one_unit():
    dev = require_gpu()
    # one unit of 65536 columns with a slot map: the radix steps spread over
    # the key slices keep their histograms, state and counts in the array;
    # then a shorter row of two units, whose steps must not read stale state
    s = _scores(dev, 1, 65536, 5)
    dead = torch.zeros(65536, dtype=torch.int32, device=dev)
    dead[::13] = 7
    ref, got = _both(dev, s, k_total=8192, n_sink=4, n_recent=64, slot_map=dead, dead_slot=7)
    _same(ref, got)
    s2 = _scores(dev, 2, 40001, 6)
    ref, got = _both(dev, s2, k_total=3000, n_sink=2, n_recent=9)
    _same(ref, got)


def test_noalloc_select_rejects_calls_beyond_its_scratch():
    dev = require_gpu()
    # 4 bytes per score: 17M scores need more than the 64 MiB array
    U, n = 520, 32768
    assert U * n * 4 > _abi.NOALLOC_SCRATCH_BYTES
    s = torch.zeros((U, n), device=dev)
    kept = torch.empty((U, 64), dtype=torch.int32, device=dev)
    with pytest.raises(kv.KvselError) as e:
        kv.select_noalloc(s, kept, k_total=64, n_sink=1, n_recent=1, pool="avg", pool_k=3)
    assert e.value.status == _abi.KVSEL_E_WORKSPACE
    # the same call with a caller workspace is fine
    kv.select(s, kept, k_total=64, n_sink=1, n_recent=1, pool="avg", pool_k=3)
    torch.cuda.synchronize()
