"""GPU parity of kvsel_free_list (IntentKV's alias-aware deallocation after
the redirect) against the oracle's free_list: the freed slot list must match
exactly."""
import numpy as np
import pytest
import torch

from oracle import materialise as om
from parity import require_gpu

import selection_score_amd as kv

pytestmark = pytest.mark.gpu


def _run(dev, sm, keep, dead, n_slots, protected_len=0, ws=None):
    N = len(sm)
    t_sm = torch.from_numpy(np.asarray(sm, dtype=np.int32)).to(dev)
    t_keep = torch.from_numpy(np.asarray(keep, dtype=np.uint8)).to(dev)
    out = torch.full((max(N, 1),), -7, dtype=torch.int32, device=dev)
    nf = torch.full((1,), -7, dtype=torch.int32, device=dev)
    ws = kv.free_list(t_sm, t_keep, dead, out, nf, n_slots=n_slots, protected_len=protected_len, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()[:N], int(nf.item()), ws


def _check(got, nf, want, N):
    assert nf == len(want)
    np.testing.assert_array_equal(got[:nf], want)
    assert np.all(got[nf:N] == -1)


def test_free_list_hand_example():
    dev = require_gpu()
    D = 99
    sm = [5, 6, 6, 7, D, 9, 5, 10, 11, 11]
    keep = [1, 0, 1, 0, 0, 0, 0, 1, 0, 0]
    got, nf, _ = _run(dev, sm, keep, D, n_slots=100)
    _check(got, nf, [7, 9, 11], 10)
    got, nf, _ = _run(dev, sm, keep, D, n_slots=100, protected_len=4)
    _check(got, nf, [9, 11], 10)


@pytest.mark.parametrize("protected_len,alias_frac", [(0, 0.0), (64, 0.05), (1000, 0.3)])
def test_free_list_session_memory_shape(protected_len, alias_frac):
    # 65536 positions over 16-token pages, the dead slot at 65536, some
    # positions already redirected and some sharing slots (aliases)
    dev = require_gpu()
    rng = np.random.default_rng(protected_len + 11)
    N, dead, n_slots = 65536, 65536, 65552
    sm = rng.permutation(N).astype(np.int64)
    n_alias = int(alias_frac * N)
    if n_alias:
        src = rng.choice(N, n_alias, replace=False)
        sm[src] = sm[rng.choice(N, n_alias)]
    sm[rng.choice(N, 2000, replace=False)] = dead
    keep = np.zeros(N, bool)
    keep[rng.choice(np.flatnonzero(sm != dead), 8192, replace=False)] = True
    got, nf, _ = _run(dev, sm, keep, dead, n_slots, protected_len)
    want = om.free_list(sm, keep, dead, protected_len)
    _check(got, nf, want, N)


def test_free_list_edges_and_workspace_reuse():
    dev = require_gpu()
    # nothing dropped
    got, nf, ws = _run(dev, [1, 2, 3], [1, 1, 1], 9, n_slots=10)
    _check(got, nf, [], 3)
    # ids outside [0, n_slots) are never freed; the same workspace serves a
    # second, larger call (the bitmaps are cleared every time)
    got, nf, ws = _run(dev, [-3, 4, 12, 4, 7], [0, 0, 0, 1, 0], 9, n_slots=10, ws=ws)
    _check(got, nf, [7], 5)
    rng = np.random.default_rng(2)
    sm = rng.integers(0, 5000, size=3000)
    keep = rng.random(3000) < 0.5
    got, nf, _ = _run(dev, sm, keep, 4999, n_slots=5000)
    _check(got, nf, om.free_list(sm, keep, 4999), 3000)
    # N = 0 writes n_free = 0
    nfree = torch.full((1,), 5, dtype=torch.int32, device=dev)
    kv.free_list(torch.zeros(0, dtype=torch.int32, device=dev), torch.zeros(0, dtype=torch.uint8, device=dev), 0,
                 torch.zeros(1, dtype=torch.int32, device=dev), nfree, n_slots=4)
    torch.cuda.synchronize()
    assert int(nfree.item()) == 0


def test_free_list_after_select_then_redirect():
    """The session-memory materialisation in order: select, the free list
    from the map before the redirect, then the redirect.  Afterwards no
    logical position refers to a freed slot."""
    dev = require_gpu()
    rng = np.random.default_rng(8)
    N, dead, n_slots, k = 8192, 8192, 8208, 1024
    sm = rng.permutation(N).astype(np.int32)
    sm[rng.choice(N, 300, replace=False)] = dead
    t_sm = torch.from_numpy(sm).to(dev)
    scores = torch.from_numpy(rng.random(N).astype(np.float32)).to(dev)[None]
    kept = torch.empty((1, k), dtype=torch.int32, device=dev)
    mask = torch.empty((1, N), dtype=torch.uint8, device=dev)
    kv.select(scores, kept, k_total=k, n_sink=4, n_recent=64, keep_mask=mask, slot_map=t_sm, dead_slot=dead)
    out = torch.empty(N, dtype=torch.int32, device=dev)
    nf = torch.empty(1, dtype=torch.int32, device=dev)
    kv.free_list(t_sm, mask[0], dead, out, nf, n_slots=n_slots, protected_len=4)
    kv.redirect(t_sm, mask[0], dead)
    torch.cuda.synchronize()
    freed = out.cpu().numpy()[: int(nf.item())]
    after = t_sm.cpu().numpy()
    want = om.free_list(sm, mask.cpu().numpy()[0].astype(bool), dead, 4)
    np.testing.assert_array_equal(freed, want)
    assert not set(freed.tolist()) & set(after.tolist())
    assert len(freed) == N - 300 - int(mask.sum().item()) - 0   # every dropped live slot is distinct here


def test_free_list_large_slot_space():
    # more slot ids than the single-workgroup LDS bitmaps hold: the
    # multi-launch path with bitmaps in the workspace
    dev = require_gpu()
    rng = np.random.default_rng(4)
    N, n_slots = 20000, (1 << 20) + 77
    dead = n_slots - 1
    sm = rng.integers(0, n_slots - 1, size=N)
    sm[rng.choice(N, 3000, replace=False)] = sm[rng.choice(N, 3000)]   # aliases
    sm[rng.choice(N, 500, replace=False)] = dead
    keep = rng.random(N) < 0.25
    keep[sm == dead] = False
    got, nf, _ = _run(dev, sm, keep, dead, n_slots, protected_len=100)
    _check(got, nf, om.free_list(sm, keep, dead, 100), N)
