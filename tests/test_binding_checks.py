"""The Python binding refuses tensors whose dtype or size does not match what
the C call will address through a raw pointer (CPU only: the checks run
before any pointer is taken)."""
import pytest
import torch

import selection_score_amd as kv


def test_keep_score_checks_types_and_shapes():
    state = torch.zeros((2, 3, 4, 10))
    keep = torch.zeros((3, 10))
    with pytest.raises(TypeError, match="n_len"):
        kv.keep_score(state, keep, torch.zeros(3, dtype=torch.int64), lam=0.5)
    with pytest.raises(ValueError, match="n_len"):
        kv.keep_score(state, keep, torch.zeros(2, dtype=torch.int32), lam=0.5)
    with pytest.raises(ValueError, match="keep"):
        kv.keep_score(state, torch.zeros((3, 9)), torch.zeros(3, dtype=torch.int32), lam=0.5)
    with pytest.raises(TypeError, match="hit"):
        kv.keep_score(state, keep, torch.zeros(3, dtype=torch.int32), lam=0.5,
                      hit=torch.zeros((3, 10), dtype=torch.bool))


def test_decode_score_checks_lse_and_counts():
    q = torch.zeros((2, 3, 8, 64), dtype=torch.bfloat16)
    pool = torch.zeros((2, 10, 16, 2, 64), dtype=torch.bfloat16)
    bt = torch.zeros((3, 4), dtype=torch.int32)
    n = torch.zeros(3, dtype=torch.int32)
    state = torch.zeros((2, 3, 2, 64))
    with pytest.raises(ValueError, match="lse"):
        kv.decode_score(q, torch.zeros((2, 3, 7)), pool, bt, n, n, state)
    with pytest.raises(ValueError, match="n_seen"):
        kv.decode_score(q, torch.zeros((2, 3, 8)), pool, bt, n, n[:2], state)
    with pytest.raises(TypeError, match="state"):
        kv.decode_score(q, torch.zeros((2, 3, 8)), pool, bt, n, n, state.double())


def test_select_compact_and_free_list_check_outputs():
    with pytest.raises(TypeError, match="scores"):
        kv.select(torch.zeros((2, 100), dtype=torch.float64), torch.zeros((2, 10), dtype=torch.int32),
                  k_total=10, n_sink=1, n_recent=1)
    with pytest.raises(ValueError, match="kept_idx"):
        kv.select(torch.zeros((2, 100)), torch.zeros((2, 9), dtype=torch.int32), k_total=10, n_sink=1,
                  n_recent=1)
    keep = torch.zeros((2, 40), dtype=torch.uint8)
    bt = torch.zeros((2, 3), dtype=torch.int32)
    pool = torch.zeros((1, 8, 16, 1, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="slot_pos"):
        kv.compact(keep, bt, pool, pool.clone(), torch.zeros((2, 47), dtype=torch.int32),
                   torch.zeros((2, 3), dtype=torch.int32), torch.zeros(2, dtype=torch.int32), block_size=16)
    with pytest.raises(TypeError, match="keep_mask"):
        kv.free_list(torch.zeros(8, dtype=torch.int32), torch.zeros(8, dtype=torch.bool), 99,
                     torch.zeros(8, dtype=torch.int32), torch.zeros(1, dtype=torch.int32), n_slots=100)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library every call raises: there is no fallback."""
    from selection_score_amd import _abi
    missing = str(tmp_path / "libkvsel.so")
    monkeypatch.setattr(_abi, "_lib", None)
    monkeypatch.setattr(_abi.load, "__defaults__", (missing,))
    with pytest.raises(RuntimeError, match="not built"):
        _abi.load()
    with pytest.raises(RuntimeError, match="not built"):
        kv.version()
