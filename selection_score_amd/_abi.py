"""ctypes mirror of include/kvsel.h and the library loader.

Struct field order and types follow the header exactly; ctypes applies the
same natural alignment as the C compiler on x86-64.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvsel.so")

KVSEL_OK, KVSEL_E_ARG, KVSEL_E_BUDGET, KVSEL_E_UNSUPPORTED, KVSEL_E_WORKSPACE, KVSEL_E_DEVICE = range(6)
STATUS_NAMES = {0: "KVSEL_OK", 1: "KVSEL_E_ARG", 2: "KVSEL_E_BUDGET", 3: "KVSEL_E_UNSUPPORTED",
                4: "KVSEL_E_WORKSPACE", 5: "KVSEL_E_DEVICE"}
F32, BF16, F16 = 0, 1, 2
SCORE_WINDOW, SCORE_MEMORY, SCORE_BLOCK = 0, 1, 2
AGG = {"sum": 0, "mean": 1, "max": 2}
POOL = {"none": 0, "avg": 1, "max": 2}
REDUCE = {"per_unit": 0, "global": 1}
ROPE = {"none": 0, "raw": 1, "delta": 2}
STYLE = {"half": 0, "interleaved": 1}
GATHER_FRESH, GATHER_INCREMENTAL = 0, 1

c_i32, c_i64, c_u32, c_f32, c_f64, c_vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                           ctypes.c_float, ctypes.c_double, ctypes.c_void_p)


class ScoreArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_u32), ("mode", c_i32), ("q_dtype", c_i32), ("k_dtype", c_i32),
        ("L", c_i32), ("Hq", c_i32), ("Hkv", c_i32), ("D", c_i32),
        ("W", c_i32), ("S", c_i32), ("N", c_i64),
        ("q", c_vp), ("k", c_vp),
        ("page_table", c_vp), ("page_size", c_i32), ("n_sink", c_i32), ("n_recent", c_i32),
        ("pool_pages", c_i64), ("slot_map", c_vp), ("dead_slot", c_i64),
        ("n_begin", c_i64), ("n_count", c_i64), ("qbar", c_vp), ("qbar_valid", c_i32),
        ("causal", c_i32), ("lse_in", c_vp), ("lse_out", c_vp),
        ("head_agg", c_i32), ("row_agg", c_i32), ("reduce", c_i32),
        ("pool", c_i32), ("pool_k", c_i32), ("scale", c_f32), ("scores", c_vp),
        ("admit", c_vp), ("tile_mask", c_vp),
    ]


class SelectArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_u32), ("U", c_i32), ("n", c_i64), ("row_stride", c_i64),
        ("scores", c_vp), ("base", c_i64), ("n_total", c_i64),
        ("k_total", c_i32), ("n_sink", c_i32), ("n_recent", c_i32),
        ("slot_map", c_vp), ("dead_slot", c_i64),
        ("cand_score", c_vp), ("cand_idx", c_vp), ("cand_count", c_vp), ("finalize", c_i32),
        ("kept_idx", c_vp), ("keep_mask", c_vp), ("n_kept", c_vp),
        ("pool", c_i32), ("pool_k", c_i32),
        ("tile_mask", c_vp), ("admit", c_vp),
    ]


class GatherArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_u32), ("mode", c_i32), ("U", c_i32), ("D", c_i32), ("dtype", c_i32),
        ("bt", c_i32), ("k", c_i32),
        ("src_k", c_vp), ("src_v", c_vp), ("src_offsets", c_vp), ("src_unit_stride", c_i64),
        ("src_rows", c_i64), ("idx", c_vp), ("n_idx", c_vp), ("dst_k", c_vp), ("dst_v", c_vp),
        ("rope", c_i32), ("style", c_i32), ("rotary_dim", c_i32), ("theta", c_f64), ("pos0", c_i64),
        ("prev_idx", c_vp), ("prev_page", c_vp), ("pool_k", c_vp), ("pool_v", c_vp),
        ("pool_pages", c_i64), ("page_table", c_vp), ("n_miss", c_vp),
        ("staged_k", c_vp), ("staged_v", c_vp), ("staged_cap", c_i64), ("hit_raw", c_i32), ("reserved", c_i32),
    ]


class RedirectArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_u32), ("N", c_i64), ("slot_map", c_vp), ("keep_mask", c_vp),
        ("dead_slot", c_i64), ("k_pool", c_vp), ("v_pool", c_vp),
        ("L", c_i32), ("Hkv", c_i32), ("D", c_i32), ("dtype", c_i32), ("pool_slots", c_i64),
        ("kept_idx", c_vp), ("k", c_i32),
    ]


class MemUpdArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_u32), ("L", c_i32), ("Hq", c_i32), ("D", c_i32), ("W", c_i32),
        ("q_dtype", c_i32), ("q_turn", c_vp), ("M", c_vp), ("decay", c_f32),
    ]


class IndexArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_u32), ("U", c_i32), ("D", c_i32), ("dtype", c_i32), ("bt", c_i32),
        ("src_k", c_vp), ("src_offsets", c_vp), ("src_unit_stride", c_i64), ("src_rows", c_i64),
        ("NB", c_i64), ("b_begin", c_i64), ("b_count", c_i64), ("mu", c_vp),
    ]


class FreeListArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_u32), ("reserved", c_i32), ("N", c_i64), ("slot_map", c_vp), ("keep_mask", c_vp),
        ("dead_slot", c_i64), ("protected_len", c_i64), ("n_slots", c_i64), ("free_slots", c_vp),
        ("n_free", c_vp),
    ]


class CompactArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_u32), ("R", c_i32), ("L", c_i32), ("Hkv", c_i32), ("D", c_i32), ("dtype", c_i32),
        ("block_size", c_i32), ("Y", c_i32), ("reserved", c_i32), ("N", c_i64), ("pool_blocks", c_i64),
        ("keep_mask", c_vp), ("block_table", c_vp), ("k_pool", c_vp), ("v_pool", c_vp), ("slot_pos", c_vp),
        ("freed_blocks", c_vp), ("n_freed", c_vp),
    ]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_u32), ("Ra", c_i32), ("R", c_i32), ("L", c_i32), ("Hq", c_i32), ("Hkv", c_i32),
        ("D", c_i32), ("dtype", c_i32), ("block_size", c_i32), ("Y", c_i32), ("scale", c_f32),
        ("n_cap", c_i64), ("pool_blocks", c_i64), ("req", c_vp), ("q", c_vp), ("lse", c_vp), ("k_pool", c_vp),
        ("block_table", c_vp), ("n_ctx", c_vp), ("n_seen", c_vp), ("state", c_vp),
    ]


class KeepScoreArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", c_u32), ("Rc", c_i32), ("R", c_i32), ("L", c_i32), ("Hkv", c_i32), ("reserved", c_i32),
        ("n_cap", c_i64), ("lam", c_f32), ("top_p", c_f32), ("req", c_vp), ("n_len", c_vp), ("state", c_vp),
        ("keep_score", c_vp), ("attn_score", c_vp), ("hit", c_vp),
    ]


EXPORTS = ["kvsel_version", "kvsel_last_error", "kvsel_score_workspace", "kvsel_score",
           "kvsel_select_workspace", "kvsel_select", "kvsel_gather_workspace", "kvsel_gather_rerope",
           "kvsel_redirect", "kvsel_memory_update", "kvsel_build_index", "kvsel_free_list_workspace",
           "kvsel_free_list", "kvsel_compact_workspace", "kvsel_compact", "kvsel_decode_score",
           "kvsel_keep_score_workspace", "kvsel_keep_score", "kvsel_select_noalloc"]
NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None


def load(path=LIB_PATH):
    """Load libkvsel.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libkvsel.so is not built (%s); run `python -m selection_score_amd.build`"
                           % path)
    lib = ctypes.CDLL(path)
    lib.kvsel_version.restype = c_i32
    lib.kvsel_version.argtypes = []
    lib.kvsel_last_error.restype = ctypes.c_char_p
    lib.kvsel_last_error.argtypes = []
    P = ctypes.POINTER
    lib.kvsel_score_workspace.argtypes = [P(ScoreArgs), P(ctypes.c_size_t)]
    lib.kvsel_score.argtypes = [P(ScoreArgs), c_vp, ctypes.c_size_t, c_vp]
    lib.kvsel_select_workspace.argtypes = [P(SelectArgs), P(ctypes.c_size_t)]
    lib.kvsel_select.argtypes = [P(SelectArgs), c_vp, ctypes.c_size_t, c_vp]
    lib.kvsel_gather_workspace.argtypes = [P(GatherArgs), P(ctypes.c_size_t)]
    lib.kvsel_gather_rerope.argtypes = [P(GatherArgs), c_vp, ctypes.c_size_t, c_vp]
    lib.kvsel_redirect.argtypes = [P(RedirectArgs), c_vp]
    lib.kvsel_memory_update.argtypes = [P(MemUpdArgs), c_vp]
    lib.kvsel_build_index.argtypes = [P(IndexArgs), c_vp]
    lib.kvsel_free_list_workspace.argtypes = [P(FreeListArgs), P(ctypes.c_size_t)]
    lib.kvsel_free_list.argtypes = [P(FreeListArgs), c_vp, ctypes.c_size_t, c_vp]
    lib.kvsel_compact_workspace.argtypes = [P(CompactArgs), P(ctypes.c_size_t)]
    lib.kvsel_compact.argtypes = [P(CompactArgs), c_vp, ctypes.c_size_t, c_vp]
    lib.kvsel_decode_score.argtypes = [P(DecodeArgs), c_vp]
    lib.kvsel_keep_score_workspace.argtypes = [P(KeepScoreArgs), P(ctypes.c_size_t)]
    lib.kvsel_keep_score.argtypes = [P(KeepScoreArgs), c_vp, ctypes.c_size_t, c_vp]
    lib.kvsel_select_noalloc.argtypes = [P(SelectArgs), c_vp]
    for name in EXPORTS[2:]:
        getattr(lib, name).restype = c_i32
    _lib = lib
    return lib
