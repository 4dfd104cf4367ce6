"""Paged KV addressing.  Test infrastructure only (see ``oracle/__init__``).

ActKV §2 (paged KV cache management): the KV pool is split into fixed-size
physical blocks of BS slots; a per-request block table maps the i-th logical
block to a physical block, so logical position j lives in physical slot
``block_table[j // BS] * BS + j % BS``.  The page prints a worked example
(BS = 2, block table [17, 9], 3 used positions) which ``tests/golden`` holds.
"""
import numpy as np


def slot_map_from_block_table(block_table, block_size, n_used):
    """Physical slot of each of the first ``n_used`` logical positions."""
    bt = np.asarray(block_table, dtype=np.int64)
    out = np.empty(n_used, dtype=np.int64)
    for j in range(n_used):
        out[j] = bt[j // block_size] * block_size + j % block_size
    return out


def logical_keys_from_pool(k_pool_layer, slot_map, page_size):
    """Keys in logical order for one layer.

    ``k_pool_layer``: [P][page_size][Hkv][D]; ``slot_map``: [N] physical slots.
    Returns [Hkv][N][D] (float64).
    """
    s = np.asarray(slot_map, dtype=np.int64)
    k = np.asarray(k_pool_layer, dtype=np.float64)
    rows = k[s // page_size, s % page_size]          # [N][Hkv][D]
    return np.transpose(rows, (1, 0, 2))
