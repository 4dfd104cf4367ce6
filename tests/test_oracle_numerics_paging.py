"""Pins for the oracle's rounding helpers and paged addressing (CPU only)."""
import json
import os

import numpy as np
import torch

from oracle import numerics, paging
from oracle.materialise import sentinel_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_slot_map_worked_example():
    g = _load("slot_map_example.json")
    got = paging.slot_map_from_block_table(g["block_table"], g["block_size"], g["seqused_k"])
    assert got.tolist() == g["slot_map"]


def test_sentinel_bits_match_fixture():
    g = _load("sentinel_bits.json")
    kb, vb = sentinel_rows("bf16", 4)
    kh, vh = sentinel_rows("f16", 4)
    assert np.all(kb == g["bf16"]["value"]) and np.all(vb == 0)
    assert np.all(kh == g["f16"]["value"]) and np.all(vh == 0)
    assert int(numerics.bf16_bits(kb)[0]) == int(g["bf16"]["bits"], 16)
    assert int(numerics.f16_bits(kh)[0]) == int(g["f16"]["bits"], 16)


def test_bf16_halfway_cases_round_to_even():
    one = 1.0
    assert numerics.round_to_bf16(one + 2.0 ** -8) == one                 # tie -> even (down)
    assert numerics.round_to_bf16(one + 3 * 2.0 ** -8) == one + 2.0 ** -6  # tie -> even (up)
    assert numerics.round_to_bf16(-(one + 2.0 ** -8)) == -one
    # a single rounding from float64: a float32 intermediate would give 1.0
    assert numerics.round_to_bf16(one + 2.0 ** -8 + 2.0 ** -40) == one + 2.0 ** -7
    assert np.signbit(numerics.round_to_bf16(-0.0))
    assert numerics.round_to_bf16(3.5e38) == np.inf


def test_bf16_matches_torch_on_float32_values():
    # for inputs already in float32 a direct rounding and torch's RNE cast agree
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(1000) * 1e-39]).astype(np.float32)
    ours = numerics.round_to_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_f16_matches_numpy_half():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000)
    ours = numerics.round_to_f16(x)
    ref = x.astype(np.float16).astype(np.float64)
    np.testing.assert_array_equal(ours, ref)
    assert numerics.round_to_f16(65519.0) == 65504.0
    assert numerics.round_to_f16(65520.0) == np.inf


def test_logical_keys_through_pages():
    # pages stored in a permuted physical order read back in logical order
    rng = np.random.default_rng(2)
    ps, n_pages, hkv, d = 4, 5, 2, 3
    logical = rng.standard_normal((hkv, n_pages * ps, d))
    perm = rng.permutation(n_pages)
    pool = np.zeros((n_pages, ps, hkv, d))
    for lp in range(n_pages):
        for o in range(ps):
            pool[perm[lp], o] = logical[:, lp * ps + o]
    slots = paging.slot_map_from_block_table(perm, ps, n_pages * ps)
    np.testing.assert_array_equal(paging.logical_keys_from_pool(pool, slots, ps), logical)
