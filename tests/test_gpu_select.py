"""GPU parity of kvsel_select against the oracle's select_topk (bit-exact on
identical float32 scores)."""
import numpy as np
import pytest
import torch

from oracle import select as osel
from parity import check_selection, require_gpu

import selection_score_amd as kv

pytestmark = pytest.mark.gpu


def _scores(rng, U, n, ties=False):
    s = rng.standard_normal((U, n)).astype(np.float32)
    if ties:
        # coarse values: many exact ties, some -0.0 / +0.0
        s = np.round(s * 4) / 4
        z = rng.random((U, n)) < 0.05
        s[z] = np.where(rng.random(int(z.sum())) < 0.5, -0.0, 0.0)
    return s


def _run(dev, s, k, n_sink, n_recent, slot_map=None, dead=0):
    U, n = s.shape
    st = torch.from_numpy(s).to(dev)
    kept = torch.full((U, k), -7, dtype=torch.int32, device=dev)
    mask = torch.zeros((U, n), dtype=torch.uint8, device=dev)
    nk = torch.zeros(U, dtype=torch.int32, device=dev)
    sm = None if slot_map is None else torch.from_numpy(slot_map.astype(np.int32)).to(dev)
    kv.select(st, kept, k_total=k, n_sink=n_sink, n_recent=n_recent, keep_mask=mask, n_kept=nk,
              slot_map=sm, dead_slot=dead)
    torch.cuda.synchronize()
    return kept.cpu().numpy(), mask.cpu().numpy(), nk.cpu().numpy()


def _check(s, kept, mask, nk, k, n_sink, n_recent, alive=None):
    for u in range(s.shape[0]):
        ok, om = osel.select_topk(s[u], k, n_sink, n_recent, alive)
        assert nk[u] == len(ok), (u, nk[u], len(ok))
        np.testing.assert_array_equal(kept[u, : len(ok)], ok)
        assert np.all(kept[u, len(ok):] == -1)
        np.testing.assert_array_equal(mask[u].astype(bool), om)


@pytest.mark.parametrize("U,n,k,n_sink,n_recent,ties", [
    (3, 1000, 100, 4, 64, False),        # ragged, several tiles of 64 (256-thread single launch)
    (5, 2048, 512, 4, 64, True),         # ties and signed zeros; the longest 256-thread row
    (2, 5000, 700, 3, 9, True),          # few units of a short row: the 1024-thread single launch
    (4, 32768, 8192, 4, 256, False),     # 32 keys per thread in registers, full per-unit size
    (2, 40000, 5000, 3, 7, True),        # beyond 32 keys per thread: keys streamed from the workspace
    (2, 65536, 20000, 4, 64, True),      # the session-memory unit size
    (1, 70001, 9000, 2, 9, True),        # a ragged last slice
    (1, 7, 3, 1, 1, True),
])
def test_select_matches_oracle(U, n, k, n_sink, n_recent, ties):
    dev = require_gpu()
    rng = np.random.default_rng(100 + n)
    s = _scores(rng, U, n, ties)
    kept, mask, nk = _run(dev, s, k, n_sink, n_recent)
    _check(s, kept, mask, nk, k, n_sink, n_recent)


@pytest.mark.parametrize("case", ["plateau", "all", "forced_only", "dead", "units8", "units9"])
def test_select_long_rows_of_few_units(case):
    """Rows longer than 32768 over at most 8 units run the radix steps spread
    over the 4096-column slices (one launch per step): a plateau of equal
    keys spanning every slice that the budget cuts part-way (ties ranked by
    position across slices), a budget that keeps every candidate, a budget
    the forced set fills exactly, dead slots over several units, and 8 and 9
    units (the last takes the single-workgroup path).  Kept list, keep mask
    and count bit for bit against select_topk."""
    dev = require_gpu()
    rng = np.random.default_rng(len(case) + 900)
    U, n, k, n_sink, n_recent = 2, 50001, 6000, 4, 64
    slot_map, alive, dead = None, None, 0
    s = rng.standard_normal((U, n)).astype(np.float32)
    if case == "plateau":
        k = 30000                                            # the cut falls in slice 9 of 13
        s = np.where(rng.random((U, n)) < 0.7, np.float32(0.5), s).astype(np.float32)
        s[:, ::97] = 2.0                                     # a few above the plateau
    elif case == "all":
        k = n + 10
    elif case == "forced_only":
        k, n_sink, n_recent = 100, 40, 60
    elif case == "dead":
        U, dead = 3, n
        slot_map = np.arange(n, dtype=np.int64)
        slot_map[rng.choice(n, n // 7, replace=False)] = dead
        slot_map[[0, 5, n - 1]] = dead                       # dead inside the forced set too
        alive = slot_map != dead
    elif case == "units8":
        U, n = 8, 40000
        s = (np.round(rng.standard_normal((U, n)) * 4) / 4).astype(np.float32)
    else:
        U, n = 9, 40000
        s = (np.round(rng.standard_normal((U, n)) * 4) / 4).astype(np.float32)
    kept, mask, nk = _run(dev, s, k, n_sink, n_recent, slot_map, dead)
    _check(s, kept, mask, nk, k, n_sink, n_recent, alive)


def test_select_global_unit_with_dead_slots():
    # the session-memory shape: one unit of 65536 with redirected positions
    dev = require_gpu()
    rng = np.random.default_rng(7)
    n, k, dead = 65536, 8192, 65536
    s = _scores(rng, 1, n)
    slot_map = rng.permutation(n).astype(np.int64)
    dead_pos = rng.choice(n, 3000, replace=False)
    slot_map[dead_pos] = dead
    dead_pos = np.concatenate([dead_pos, [0, n - 1]])  # dead positions inside the forced set too
    slot_map[[0, n - 1]] = dead
    alive = slot_map != dead
    kept, mask, nk = _run(dev, s, k, 4, 64, slot_map, dead)
    _check(s, kept, mask, nk, k, 4, 64, alive)


@pytest.mark.parametrize("k,n_sink,n_recent", [(2048, 5, 5), (10, 4, 6), (3000, 0, 0)])
def test_select_edge_budgets(k, n_sink, n_recent):
    dev = require_gpu()
    rng = np.random.default_rng(k)
    s = _scores(rng, 2, 2048, ties=True)
    kept, mask, nk = _run(dev, s, k, n_sink, n_recent)
    _check(s, kept, mask, nk, k, n_sink, n_recent)


def test_select_all_dead_and_empty():
    dev = require_gpu()
    n = 300
    s = np.zeros((1, n), np.float32)
    slot_map = np.full(n, 9, np.int64)
    kept, mask, nk = _run(dev, s, 50, 2, 2, slot_map, 9)
    assert nk[0] == 0 and np.all(kept == -1) and not mask.any()
    # U = 0 is a no-op
    kv.select(torch.zeros((0, 10), device=dev), torch.zeros((0, 4), dtype=torch.int32, device=dev),
              k_total=4, n_sink=0, n_recent=0)
    # n = 0 with enough units for the single-launch path: the scores are an
    # empty (NULL) buffer, nothing may be read, every unit keeps nothing
    for U in (128, 300):
        kept = torch.full((U, 6), 7, dtype=torch.int32, device=dev)
        nk = torch.full((U,), 5, dtype=torch.int32, device=dev)
        kv.select(torch.empty((U, 0), device=dev), kept, k_total=6, n_sink=2, n_recent=2, n_kept=nk)
        torch.cuda.synchronize()
        assert torch.all(kept == -1) and torch.all(nk == 0)


def test_select_budget_error():
    dev = require_gpu()
    s = torch.zeros((1, 100), device=dev)
    kept = torch.zeros((1, 8), dtype=torch.int32, device=dev)
    with pytest.raises(kv.KvselError) as e:
        kv.select(s, kept, k_total=8, n_sink=5, n_recent=5)
    assert e.value.status == 2


@pytest.mark.parametrize("n,tile,k", [(100000, 30000, 4096), (70001, 65536, 4096), (5000, 977, 300)])
def test_select_tiled_equals_untiled(n, tile, k):
    dev = require_gpu()
    rng = np.random.default_rng(n)
    U = 3
    s = _scores(rng, U, n, ties=True)
    st = torch.from_numpy(s).to(dev)
    cs = torch.zeros((U, k), dtype=torch.float32, device=dev)
    ci = torch.zeros((U, k), dtype=torch.int32, device=dev)
    cc = torch.zeros(U, dtype=torch.int32, device=dev)
    kept = torch.full((U, k), -7, dtype=torch.int32, device=dev)
    nk = torch.zeros(U, dtype=torch.int32, device=dev)
    for b in range(0, n, tile):
        e = min(n, b + tile)
        kv.select(st[:, b:e], kept, k_total=k, n_sink=1, n_recent=4, n_total=n, base=b,
                  cand_score=cs, cand_idx=ci, cand_count=cc, finalize=(e == n), n_kept=nk)
    torch.cuda.synchronize()
    kept, nk = kept.cpu().numpy(), nk.cpu().numpy()
    for u in range(U):
        ok, _ = osel.select_topk(s[u], k, 1, 4)
        assert nk[u] == len(ok)
        np.testing.assert_array_equal(kept[u, : len(ok)], ok)


def pack_tile(x, thr):
    """Packed tile form of dense rows x [U][m] under per-row thresholds thr
    [U] (NaN admits every column): per 256-column chunk the admitted scores
    in column order at the chunk's start, every other position NaN (a read
    of one would disturb the selection), and the uint64 mask words as int64."""
    U, m = x.shape
    adm = np.where(np.isnan(thr)[:, None], True, x > thr[:, None])
    packed = np.full((U, m), np.nan, np.float32)
    for c0 in range(0, m, 256):
        a = adm[:, c0:c0 + 256]
        for u in range(U):
            v = x[u, c0:c0 + 256][a[u]]
            packed[u, c0:c0 + len(v)] = v
    n_words = (m + 63) // 64
    bits = np.zeros((U, n_words * 64), bool)
    bits[:, :m] = adm
    words = (bits.reshape(U, n_words, 64).astype(np.uint64) << np.arange(64, dtype=np.uint64)).sum(axis=2,
                                                                                                  dtype=np.uint64)
    return packed, words.view(np.int64), adm


def _tiled(dev, s, k, n_sink, n_recent, tile, slot_map=None, dead_slot=0, stride_pad=0, packed=None):
    """Tiled selection of every row of s (with an optional slot map), tiles
    of `tile` columns in ascending order; the rows may sit in a wider
    buffer (stride_pad extra columns) so that tile rows are misaligned.
    packed: None (dense tiles), "exact" (every tile after the first packed
    under the threshold the previous call wrote, which is checked against
    the running set), or "low" (packed under lower thresholds: NaN on even
    rows, the next float below on odd rows)."""
    U, n = s.shape
    buf = torch.zeros((U, n + stride_pad), dtype=torch.float32, device=dev)
    buf[:, :n] = torch.from_numpy(s).to(dev)
    cs = torch.full((U, k), 123.0, device=dev)
    ci = torch.full((U, k), -9, dtype=torch.int32, device=dev)
    cc = torch.zeros(U, dtype=torch.int32, device=dev)
    kept = torch.full((U, k), -7, dtype=torch.int32, device=dev)
    nk = torch.zeros(U, dtype=torch.int32, device=dev)
    sm = None if slot_map is None else torch.from_numpy(slot_map.astype(np.int32)).to(dev)
    admit = torch.full((U,), 5.0, device=dev) if packed else None
    alive = np.ones(n, bool) if slot_map is None else slot_map != dead_slot
    room = k - int((osel.forced_mask(n, n_sink, n_recent) & alive).sum())
    for b in range(0, n, tile):
        e = min(n, b + tile)
        rows, mask = buf[:, b:e], None
        if packed and b > 0:
            thr = admit.cpu().numpy()
            # the threshold is the running set's smallest score once it is full
            cnt, cand = cc.cpu().numpy(), cs.cpu().numpy()
            for u in range(U):
                if cnt[u] == room and room > 0:
                    assert thr[u] == cand[u, :room].min(), (u, thr[u])
                else:
                    assert np.isnan(thr[u])
            if packed == "low":
                thr = np.where(np.arange(U) % 2 == 0, np.nan, np.nextafter(thr, np.float32(-np.inf)))
            pk, words, _ = pack_tile(s[:, b:e], thr.astype(np.float32))
            pbuf = torch.zeros((U, e - b + stride_pad), dtype=torch.float32, device=dev)
            pbuf[:, :e - b] = torch.from_numpy(pk).to(dev)
            rows, mask = pbuf[:, :e - b], torch.from_numpy(words).to(dev)
        kv.select(rows, kept, k_total=k, n_sink=n_sink, n_recent=n_recent, n_total=n, base=b,
                  cand_score=cs, cand_idx=ci, cand_count=cc, finalize=(e == n), n_kept=nk, slot_map=sm,
                  dead_slot=dead_slot, tile_mask=mask, admit=admit if e < n else None)
    torch.cuda.synchronize()
    return kept.cpu().numpy(), nk.cpu().numpy()


@pytest.mark.parametrize("packed", [None, "exact", "low"])
@pytest.mark.parametrize("case", ["equal", "ascending", "descending", "coarse", "dead", "k8192", "misaligned",
                                  "bin5k", "bin9k"])
def test_select_tiled_hard_cases(case, packed):
    """Tiles whose survivors overflow the LDS set (the first tile; rising
    scores), plateaus of equal keys wider than any LDS set (every column
    ranked by index), nothing surviving after the first tile, dead slots,
    the largest budget, and tile rows that are not 16-byte aligned; with
    dense tiles, and with tiles packed under the admission threshold the
    previous call wrote (or a lower one).  bin5k / bin9k: normal scores
    whose first 65536-column tile holds about 5000 / 8750 columns at or
    above the top-12-bit bin of its threshold (3 + 0.7 z: the bin starts at
    4.0 = 1.43 sigma; 4 + 0.9 z: at 5.0 = 1.11 sigma), more than a set
    beside a full running set holds, fewer / more than the first tile's
    (whose running set is empty).  The tiled result must equal the untiled
    oracle selection bit for bit."""
    dev = require_gpu()
    rng = np.random.default_rng(len(case))
    U, n, tile, k, n_sink, n_recent = 3, 70000, 16384, 4096, 4, 64
    slot_map, alive, dead_slot, pad = None, None, 0, 0
    if case == "equal":
        s = np.full((U, n), 0.75, np.float32)
    elif case == "ascending":
        s = np.tile(np.linspace(-3, 3, n, dtype=np.float32), (U, 1))
    elif case == "descending":
        s = np.tile(np.linspace(3, -3, n, dtype=np.float32), (U, 1))
    elif case == "coarse":
        s = (np.round(rng.standard_normal((U, n)) * 2) / 2).astype(np.float32)
    elif case == "dead":
        s = rng.standard_normal((U, n)).astype(np.float32)
        dead_slot = 1 << 20
        slot_map = np.arange(n, dtype=np.int64)
        slot_map[rng.choice(n, n // 3, replace=False)] = dead_slot
        slot_map[[0, n - 1]] = dead_slot
        alive = slot_map != dead_slot
    elif case == "k8192":
        n, tile, k = 200000, 65536, 8192
        s = rng.standard_normal((U, n)).astype(np.float32)
    elif case in ("bin5k", "bin9k"):
        n, tile = 140000, 65536
        mean, sd = (3.0, 0.7) if case == "bin5k" else (4.0, 0.9)
        s = (mean + sd * rng.standard_normal((U, n))).astype(np.float32)
    else:
        n, tile, pad = 50001, 10001, 3
        s = rng.standard_normal((U, n)).astype(np.float32)
    got, nk = _tiled(dev, s, k, n_sink, n_recent, tile, slot_map, dead_slot, pad, packed)
    for u in range(U):
        ok, _ = osel.select_topk(s[u].astype(np.float64), k, n_sink, n_recent, alive)
        assert nk[u] == len(ok), case
        np.testing.assert_array_equal(got[u, : len(ok)], ok, err_msg=case)
        assert np.all(got[u, len(ok):] == -1)


@pytest.mark.parametrize("pool,n", [("max", 4099), ("avg", 4097), ("max", 40000)])
def test_select_pooled_slices(pool, n):
    """Pooling across the 4096-column slices of the key preparation (halo at
    both slice edges, ragged last slice), against pool1d + select_topk."""
    from oracle import numerics
    from oracle import score as osc
    dev = require_gpu()
    rng = np.random.default_rng(7 + n)
    U, k, n_sink, n_recent = 3, n // 5, 4, 64
    s = rng.standard_normal((U, n)).astype(np.float32)
    st = torch.from_numpy(s).to(dev)
    kept = torch.empty((U, k), dtype=torch.int32, device=dev)
    kv.select(st, kept, k_total=k, n_sink=n_sink, n_recent=n_recent, pool=pool, pool_k=7)
    torch.cuda.synchronize()
    got = kept.cpu().numpy()
    for u in range(U):
        # max-pooling is exact in float32; the average may differ from the
        # float64 mean by rounding, so near-ties follow the shared rule
        pooled = numerics.round_to_f32(osc.pool1d(s[u].astype(np.float64), pool, 7))
        verdict = check_selection(got[u], pooled, k, n_sink, n_recent, what="unit %d" % u)
        if pool == "max":
            assert verdict == "exact"



@pytest.mark.parametrize("U,n,k,pool,pool_k,ties,dead", [
    (130, 5000, 700, "none", 1, True, False),      # ragged rows, exact ties and signed zeros
    (128, 32768, 8192, "none", 1, False, True),    # the per-unit maximum with dead positions
    (129, 4099, 800, "max", 7, False, False),      # max-pool halo at every wavefront segment edge
    (130, 3001, 500, "avg", 5, False, True),
    (128, 2000, 300, "max", 1, True, False),       # a window of one
    (128, 6000, 900, "avg", 255, False, False),    # the widest window
    (128, 2000, 300, "max", 3, True, False),       # max windows of 3 to 9 in registers: short rows,
    (131, 7001, 900, "max", 5, False, False),      # ties, ragged rows, every doubling depth and
    (128, 32768, 8192, "max", 9, False, False),    # second offset, the longest rows
    (128, 9000, 1000, "max", 11, False, False),    # a window of 11 keeps the two launches
    (128, 2000, 300, "avg", 7, True, False),       # average windows in registers on short rows
    (129, 1500, 200, "avg", 9, False, False),
])
def test_select_many_units(U, n, k, pool, pool_k, ties, dead):
    """Many units: unpooled rows (and windows of one), max-pooled rows with
    windows up to 9, and average-pooled rows of at most 2048 columns with
    windows up to 9, without a slot map, take the single-launch path where
    each unit's workgroup makes its own keys; other pooled rows and dead
    slots keep the two launches.  Against pool1d + select_topk."""
    from oracle import numerics
    from oracle import score as osc
    dev = require_gpu()
    rng = np.random.default_rng(U * 7 + n)
    n_sink, n_recent = 4, 64
    s = _scores(rng, U, n, ties)
    slot_map, alive, dead_slot = None, None, n
    if dead:
        slot_map = np.arange(n, dtype=np.int64)
        slot_map[rng.choice(n, n // 10, replace=False)] = dead_slot
        slot_map[[1, n - 2]] = dead_slot                 # dead inside the forced set too
        alive = slot_map != dead_slot
    st = torch.from_numpy(s).to(dev)
    kept = torch.full((U, k), -7, dtype=torch.int32, device=dev)
    nk = torch.zeros(U, dtype=torch.int32, device=dev)
    mask = torch.zeros((U, n), dtype=torch.uint8, device=dev)
    sm = None if slot_map is None else torch.from_numpy(slot_map.astype(np.int32)).to(dev)
    kv.select(st, kept, k_total=k, n_sink=n_sink, n_recent=n_recent, keep_mask=mask, n_kept=nk,
              slot_map=sm, dead_slot=dead_slot, pool=pool, pool_k=pool_k)
    torch.cuda.synchronize()
    got, nk, mask = kept.cpu().numpy(), nk.cpu().numpy(), mask.cpu().numpy()
    if pool == "none" or pool_k == 1:
        _check(s, got, mask, nk, k, n_sink, n_recent, alive)
        return
    pooled = numerics.round_to_f32(osc.pool1d(s.astype(np.float64), pool, pool_k))
    for u in range(U):
        verdict = check_selection(got[u], pooled[u], k, n_sink, n_recent, alive, what="unit %d" % u)
        if pool == "max":
            assert verdict == "exact"
        ok, om = osel.select_topk(pooled[u].astype(np.float64), k, n_sink, n_recent, alive)
        assert nk[u] == len(ok)
        assert mask[u].sum() == len(ok)
        np.testing.assert_array_equal(np.flatnonzero(mask[u]), np.sort(got[u][got[u] >= 0]))
