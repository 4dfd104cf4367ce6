"""kvsel: attention-score-driven KV-cache selection on AMD MI355X (gfx950).

The compute lives in ``libkvsel.so`` (hand-written HIP kernels behind the C
ABI of ``include/kvsel.h``); this package is a thin ctypes binding plus the
seeded synthetic workload generators.  Importing the binding functions loads
the library lazily and raises if it has not been built.
"""
from .kvsel import (KvselError, build_index, compact, decode_score, free_list, keep_score, gather_incremental, gather_rerope, memory_update, redirect,
                    score_block, score_memory, score_window, select, select_noalloc, version)

__all__ = ["KvselError", "build_index", "compact", "decode_score", "free_list", "keep_score", "gather_incremental", "gather_rerope", "memory_update", "redirect",
           "score_block", "score_memory", "score_window", "select", "select_noalloc", "version"]
