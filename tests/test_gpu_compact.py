"""GPU parity of kvsel_compact (ActKV's in-place tail compaction of paged
KV) against the oracle's tail_compact: slot positions, freed blocks and the
pools after the copies must match exactly (the copies move bits)."""
import numpy as np
import pytest
import torch

from oracle import materialise as om
from parity import require_gpu

import selection_score_amd as kv

pytestmark = pytest.mark.gpu


def _run_and_check(dev, keep, bt, bs, L, Hkv, D, P, dtype, seed=0):
    R, N = keep.shape
    Y = bt.shape[1]
    g = torch.Generator().manual_seed(seed)
    k_pool = torch.randn((L, P, bs, Hkv, D), generator=g).to(dtype)
    v_pool = torch.randn((L, P, bs, Hkv, D), generator=g).to(dtype)
    k0, v0 = k_pool.clone(), v_pool.clone()
    kd, vd = k_pool.to(dev), v_pool.to(dev)
    slot_pos = torch.full((R, Y * bs), -7, dtype=torch.int32, device=dev)
    freed = torch.full((R, Y), -7, dtype=torch.int32, device=dev)
    nfr = torch.full((R,), -7, dtype=torch.int32, device=dev)
    kv.compact(torch.from_numpy(keep.astype(np.uint8)).to(dev), torch.from_numpy(bt.astype(np.int32)).to(dev),
               kd, vd, slot_pos, freed, nfr, block_size=bs)
    torch.cuda.synchronize()
    got_k, got_v = kd.cpu(), vd.cpu()
    want_k, want_v = k0.clone(), v0.clone()
    sp, fr, nf = slot_pos.cpu().numpy(), freed.cpu().numpy(), nfr.cpu().numpy()
    for r in range(R):
        for l in range(L):
            # bit patterns through the oracle: view the rows as int16 / int32 so
            # the copies compare bit for bit
            ib = torch.int32 if dtype == torch.float32 else torch.int16
            kp, vp, pos, fb = om.tail_compact(keep[r], bt[r], bs, want_k[l].view(ib).numpy(),
                                              want_v[l].view(ib).numpy())
            want_k[l] = torch.from_numpy(kp).view(dtype)
            want_v[l] = torch.from_numpy(vp).view(dtype)
        np.testing.assert_array_equal(sp[r], pos)
        assert nf[r] == len(fb)
        np.testing.assert_array_equal(fr[r, : len(fb)], fb)
        assert np.all(fr[r, len(fb):] == -1)
    ib = torch.int32 if dtype == torch.float32 else torch.int16
    assert torch.equal(got_k.view(ib), want_k.view(ib))
    assert torch.equal(got_v.view(ib), want_v.view(ib))


def test_compact_hand_example():
    dev = require_gpu()
    keep = np.zeros((1, 14), bool); keep[0, [0, 3, 6, 9, 10, 13]] = True
    bt = np.array([[7, 2, 9, 5]])
    _run_and_check(dev, keep, bt, bs=4, L=2, Hkv=1, D=8, P=10, dtype=torch.bfloat16)


@pytest.mark.parametrize("dtype,Hkv,D,L", [(torch.bfloat16, 8, 128, 2), (torch.float16, 2, 64, 3),
                                           (torch.float32, 1, 64, 1)])
def test_compact_requests_match_oracle(dtype, Hkv, D, L):
    # four requests of the Table-1 kind (6K positions in 16-slot blocks) with
    # different kept fractions, a ragged request, an all-kept and an all-dropped one
    dev = require_gpu()
    rng = np.random.default_rng(D + L)
    bs, Y = 16, 384
    N = Y * bs
    R = 6
    keep = np.zeros((R, N), bool)
    for r, frac in enumerate([2 / 3, 0.25, 0.9, 0.5]):
        keep[r] = rng.random(N) < frac
        keep[r, -256:] = True                           # recent entries, as a selection forces
    keep[1, N - 5:] = False                             # ragged tail inside the last block
    keep[4] = True
    keep[5] = False
    P = R * Y + 40
    bt = rng.permutation(P)[: R * Y].reshape(R, Y)
    _run_and_check(dev, keep, bt, bs, L, Hkv, D, P, dtype, seed=D)


def test_compact_partial_last_block_and_no_ops():
    dev = require_gpu()
    rng = np.random.default_rng(1)
    bs, Y, N = 16, 10, 150                              # 10 slots of the last block are empty
    keep = rng.random((2, N)) < 0.55
    bt = rng.permutation(40)[:20].reshape(2, Y)
    _run_and_check(dev, keep, bt, bs, L=1, Hkv=2, D=64, P=40, dtype=torch.bfloat16)
    # R = 0: nothing is enqueued
    e = torch.zeros((0, 5), dtype=torch.uint8, device=dev)
    pool = torch.zeros((1, 4, 16, 1, 64), dtype=torch.bfloat16, device=dev)
    kv.compact(e, torch.zeros((0, 2), dtype=torch.int32, device=dev), pool, pool.clone(),
               torch.zeros((0, 32), dtype=torch.int32, device=dev), torch.zeros((0, 2), dtype=torch.int32, device=dev),
               torch.zeros(0, dtype=torch.int32, device=dev), block_size=16)
    torch.cuda.synchronize()


def test_compact_actkv_workload_full_size_sampled():
    """The benchmarked shape: 64 requests of 6144 positions in 16-slot blocks,
    36 layers of 8 KV heads x 128 bf16, 4096 kept per request, one launch over
    all of it.  Slot positions and freed blocks are checked for every
    request; the pools bit for bit for sampled (request, layer) pairs, each
    through the oracle on that request's own blocks (a request's blocks are
    disjoint from every other's, so its compaction is local to them); blocks
    of no request must be untouched."""
    from selection_score_amd import workloads as wl
    dev = require_gpu()
    cfg = wl.CONFIGS["actkv"]
    print("compact full size: inputs", flush=True)
    inp = wl.actkv_inputs(cfg, dev)
    R, N, bs, L = cfg.S, cfg.N, cfg.page_size, cfg.L
    keep = inp["keep"].cpu().numpy().astype(bool)
    bt = inp["block_table"].cpu().numpy().astype(np.int64)
    Y = bt.shape[1]
    P = inp["k_pool"].shape[1]
    reqs, layers = (0, 29, 63), (0, 17, 35)
    spare = np.setdiff1d(np.arange(P), bt.reshape(-1))
    ib = torch.int16
    before = {}
    for l in layers:
        for name in ("k_pool", "v_pool"):
            pool = inp[name][l].view(ib)
            before[(name, l, "spare")] = pool[torch.from_numpy(spare).to(dev)].cpu()
            for r in reqs:
                before[(name, l, r)] = pool[torch.from_numpy(bt[r]).to(dev)].cpu().numpy()
    slot_pos = torch.full((R, Y * bs), -7, dtype=torch.int32, device=dev)
    freed = torch.full((R, Y), -7, dtype=torch.int32, device=dev)
    nfr = torch.full((R,), -7, dtype=torch.int32, device=dev)
    print("compact full size: launch", flush=True)
    kv.compact(inp["keep"], inp["block_table"], inp["k_pool"], inp["v_pool"], slot_pos, freed, nfr, block_size=bs)
    torch.cuda.synchronize()
    sp, fr, nf = slot_pos.cpu().numpy(), freed.cpu().numpy(), nfr.cpu().numpy()
    local = np.arange(Y)
    dummy = np.zeros((Y, bs, 1), dtype=np.int16)
    print("compact full size: plans of all requests", flush=True)
    for r in range(R):
        _, _, pos, fb = om.tail_compact(keep[r], local, bs, dummy, dummy)
        np.testing.assert_array_equal(sp[r], pos)
        assert nf[r] == len(fb)
        np.testing.assert_array_equal(fr[r, : len(fb)], bt[r][fb])
        assert np.all(fr[r, len(fb):] == -1)
    print("compact full size: sampled pools", flush=True)
    for l in layers:
        for name in ("k_pool", "v_pool"):
            pool = inp[name][l].view(ib)
            assert torch.equal(pool[torch.from_numpy(spare).to(dev)].cpu(), before[(name, l, "spare")])
            for r in reqs:
                kp, _, _, _ = om.tail_compact(keep[r], local, bs, before[(name, l, r)], before[(name, l, r)])
                got = pool[torch.from_numpy(bt[r]).to(dev)].cpu().numpy()
                np.testing.assert_array_equal(got, kp)
