"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/kvsel.h declares, the ctypes structs match the C layout,
and argument validation reports errors before any device work."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

from selection_score_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvsel.h")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(kvsel_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    lib = _abi.load()
    names = _declared_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_abi.EXPORTS)
    assert lib.kvsel_version() == 1


STRUCTS = {
    "kvsel_score_args": _abi.ScoreArgs,
    "kvsel_select_args": _abi.SelectArgs,
    "kvsel_gather_args": _abi.GatherArgs,
    "kvsel_redirect_args": _abi.RedirectArgs,
    "kvsel_memupd_args": _abi.MemUpdArgs,
    "kvsel_index_args": _abi.IndexArgs,
    "kvsel_freelist_args": _abi.FreeListArgs,
    "kvsel_compact_args": _abi.CompactArgs,
    "kvsel_decode_args": _abi.DecodeArgs,
    "kvsel_keep_score_args": _abi.KeepScoreArgs,
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_ctypes_layout_matches_header(tmp_path):
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "kvsel.h"', "int main(void) {"]
    for cname, cls in STRUCTS.items():
        lines.append('printf("%s %%zu\\n", sizeof(%s));' % (cname, cname))
        for f, _ in cls._fields_:
            lines.append('printf("%s.%s %%zu\\n", offsetof(%s, %s));' % (cname, f, cname, f))
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-I" + os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    out = dict(line.split() for line in subprocess.check_output([str(exe)], text=True).splitlines())
    for cname, cls in STRUCTS.items():
        assert int(out[cname]) == ctypes.sizeof(cls), cname
        for f, _ in cls._fields_:
            assert int(out["%s.%s" % (cname, f)]) == getattr(cls, f).offset, (cname, f)


def _select_args(**kw):
    a = _abi.SelectArgs()
    a.struct_size = ctypes.sizeof(a)
    a.U, a.n, a.row_stride, a.n_total, a.k_total = 1, 100, 100, 100, 10
    a.scores, a.kept_idx = 0x1000, 0x2000
    a.finalize = 1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _status(fn, a, *extra):
    return fn(ctypes.byref(a), *extra)


def test_select_validation_errors_without_device():
    lib = _abi.load()
    nb = ctypes.c_size_t(0)
    assert lib.kvsel_select_workspace(None, ctypes.byref(nb)) == _abi.KVSEL_E_ARG
    assert _status(lib.kvsel_select_workspace, _select_args(n_sink=6, n_recent=5), ctypes.byref(nb)) \
        == _abi.KVSEL_E_BUDGET
    assert b"exceeds" in lib.kvsel_last_error()
    # short rows: one workgroup per unit makes its own keys, no workspace
    assert _status(lib.kvsel_select_workspace, _select_args(), ctypes.byref(nb)) == _abi.KVSEL_OK
    assert nb.value == 0
    # longer rows over few units keep one 4-byte key per position in the workspace
    long_rows = dict(n=10000, row_stride=10000, n_total=10000)
    assert _status(lib.kvsel_select_workspace, _select_args(**long_rows), ctypes.byref(nb)) == _abi.KVSEL_OK
    assert nb.value >= 10000 * 4
    assert _status(lib.kvsel_select, _select_args(**long_rows), None, ctypes.c_size_t(0), None) \
        == _abi.KVSEL_E_WORKSPACE
    assert b"workspace" in lib.kvsel_last_error()
    assert _status(lib.kvsel_select, _select_args(**long_rows), ctypes.c_void_p(0x10000),
                   ctypes.c_size_t(nb.value - 1), None) == _abi.KVSEL_E_WORKSPACE
    # a max-pooled call with a short window makes its keys in registers too,
    # as does an average-pooled one over rows of at most 2048 positions; a
    # longer window, a longer average-pooled row or a slot map keeps the two launches
    for kw in (dict(pool=_abi.POOL["max"], pool_k=3), dict(pool=_abi.POOL["max"], pool_k=9),
               dict(pool=_abi.POOL["avg"], pool_k=9)):
        assert _status(lib.kvsel_select_workspace, _select_args(**kw), ctypes.byref(nb)) == _abi.KVSEL_OK
        assert nb.value == 0
    mid_rows = dict(n=3000, row_stride=3000, n_total=3000)
    for kw in (dict(pool=_abi.POOL["max"], pool_k=11), dict(pool=_abi.POOL["avg"], pool_k=11),
               dict(mid_rows, pool=_abi.POOL["avg"], pool_k=3)):
        assert _status(lib.kvsel_select_workspace, _select_args(**kw), ctypes.byref(nb)) == _abi.KVSEL_OK
        assert nb.value >= kw.get("n", 100) * 4
    # a tile of a tiled call whose running set and tile fit in LDS needs none;
    # a tile too wide for the LDS bitmap takes the two-launch path and does
    tiled = dict(cand_score=0x3000, cand_idx=0x4000, cand_count=0x5000, n=60, n_total=100, base=40)
    assert _status(lib.kvsel_select_workspace, _select_args(**tiled), ctypes.byref(nb)) == _abi.KVSEL_OK
    assert nb.value == 0
    wide = dict(tiled, n=1 << 23, n_total=(1 << 23) + 40, row_stride=1 << 23)
    assert _status(lib.kvsel_select_workspace, _select_args(**wide), ctypes.byref(nb)) == _abi.KVSEL_OK
    assert nb.value >= (1 << 23) * 4
    # a partial range without candidate buffers, or an oversize range
    assert _status(lib.kvsel_select_workspace, _select_args(n=50), ctypes.byref(nb)) == _abi.KVSEL_E_ARG
    assert _status(lib.kvsel_select_workspace, _select_args(base=60), ctypes.byref(nb)) == _abi.KVSEL_E_ARG
    assert _status(lib.kvsel_select_workspace, _select_args(struct_size=8), ctypes.byref(nb)) == _abi.KVSEL_E_ARG
    # k >= N with an oversized forced set is not a budget error
    assert _status(lib.kvsel_select_workspace, _select_args(k_total=100, n_sink=80, n_recent=80),
                   ctypes.byref(nb)) == _abi.KVSEL_OK


def _score_args(**kw):
    a = _abi.ScoreArgs()
    a.struct_size = ctypes.sizeof(a)
    a.mode, a.q_dtype, a.k_dtype = _abi.SCORE_WINDOW, _abi.BF16, _abi.BF16
    a.L, a.Hq, a.Hkv, a.D, a.W, a.S, a.N = 36, 32, 8, 128, 64, 1, 32768
    a.q, a.k, a.scores = 0x1000, 0x2000, 0x3000
    a.causal = 1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_score_validation_and_workspace_without_device():
    lib = _abi.load()
    nb = ctypes.c_size_t(0)
    assert _status(lib.kvsel_score_workspace, _score_args(), ctypes.byref(nb)) == _abi.KVSEL_OK
    # own LSE (36*32*64 floats) + per-chunk partials (36*8*16 chunks*256 rows*8 bytes)
    assert nb.value >= 36 * 32 * 64 * 4 + 36 * 8 * 16 * 256 * 8
    assert _status(lib.kvsel_score_workspace, _score_args(D=96), ctypes.byref(nb)) == _abi.KVSEL_E_UNSUPPORTED
    assert _status(lib.kvsel_score_workspace, _score_args(Hq=30), ctypes.byref(nb)) == _abi.KVSEL_E_ARG
    assert _status(lib.kvsel_score_workspace, _score_args(q=0x1004), ctypes.byref(nb)) == _abi.KVSEL_E_ARG
    assert _status(lib.kvsel_score_workspace, _score_args(pool=_abi.POOL["max"], pool_k=4),
                   ctypes.byref(nb)) == _abi.KVSEL_E_ARG
    # max aggregation on a window too large for the VALU path
    assert _status(lib.kvsel_score_workspace, _score_args(head_agg=_abi.AGG["max"], W=128),
                   ctypes.byref(nb)) == _abi.KVSEL_E_UNSUPPORTED
    # memory mode: two pages of every KV head must fit the 160 KiB of LDS
    mem = dict(mode=_abi.SCORE_MEMORY, q_dtype=_abi.F32, page_table=0x4000, pool_pages=5000, page_size=64)
    assert _status(lib.kvsel_score_workspace, _score_args(Hkv=2, **mem), ctypes.byref(nb)) == _abi.KVSEL_OK
    assert _status(lib.kvsel_score_workspace, _score_args(**mem), ctypes.byref(nb)) == _abi.KVSEL_E_UNSUPPORTED
    blk = _score_args(mode=_abi.SCORE_BLOCK, k_dtype=_abi.F16, N=1000, n_begin=900, n_count=200)
    assert _status(lib.kvsel_score_workspace, blk, ctypes.byref(nb)) == _abi.KVSEL_E_ARG
    # a score call with a too-small workspace fails before touching the device
    assert lib.kvsel_score(ctypes.byref(_score_args()), None, 0, None) == _abi.KVSEL_E_WORKSPACE


def test_packed_tile_options_are_validated_without_device():
    """The admission threshold and packed-tile mask: optional for the earlier
    struct layouts, tiled calls only (select), block mode with D 128 and
    both given together (score)."""
    lib = _abi.load()
    nb = ctypes.c_size_t(0)
    tiled = dict(cand_score=0x3000, cand_idx=0x4000, cand_count=0x5000, n=60, n_total=100, base=40)
    ok = _select_args(tile_mask=0x6000, admit=0x7000, finalize=0, **tiled)
    assert _status(lib.kvsel_select_workspace, ok, ctypes.byref(nb)) == _abi.KVSEL_OK and nb.value == 0
    assert _status(lib.kvsel_select_workspace, _select_args(tile_mask=0x6000), ctypes.byref(nb)) == _abi.KVSEL_E_ARG
    assert b"tiled" in lib.kvsel_last_error()
    assert _status(lib.kvsel_select_workspace, _select_args(admit=0x7000), ctypes.byref(nb)) == _abi.KVSEL_E_ARG
    assert _status(lib.kvsel_select_workspace, _select_args(tile_mask=0x6008, **tiled),
                   ctypes.byref(nb)) == _abi.KVSEL_E_ARG
    # a tile too wide for one workgroup's LDS takes the workspace path, which has neither option
    wide = dict(tiled, n=1 << 23, n_total=(1 << 23) + 40, row_stride=1 << 23)
    assert _status(lib.kvsel_select_workspace, _select_args(admit=0x7000, **wide),
                   ctypes.byref(nb)) == _abi.KVSEL_E_UNSUPPORTED
    # the layout that ends before tile_mask is accepted and ignores the fields' memory
    old = _select_args(tile_mask=0x6008, admit=0x7000, **tiled)
    old.struct_size = _abi.SelectArgs.tile_mask.offset
    assert _status(lib.kvsel_select_workspace, old, ctypes.byref(nb)) == _abi.KVSEL_OK
    old.struct_size = _abi.SelectArgs.tile_mask.offset - 8
    assert _status(lib.kvsel_select_workspace, old, ctypes.byref(nb)) == _abi.KVSEL_E_ARG

    blk = dict(mode=_abi.SCORE_BLOCK, k_dtype=_abi.F16, N=1000, n_begin=0, n_count=1000, S=2)
    assert _status(lib.kvsel_score_workspace, _score_args(admit=0x5000, tile_mask=0x6000, **blk),
                   ctypes.byref(nb)) == _abi.KVSEL_OK
    assert _status(lib.kvsel_score_workspace, _score_args(admit=0x5000, **blk), ctypes.byref(nb)) == _abi.KVSEL_E_ARG
    assert b"together" in lib.kvsel_last_error()
    assert _status(lib.kvsel_score_workspace, _score_args(tile_mask=0x6000, **blk),
                   ctypes.byref(nb)) == _abi.KVSEL_E_ARG
    assert _status(lib.kvsel_score_workspace, _score_args(admit=0x5000, tile_mask=0x6008, **blk),
                   ctypes.byref(nb)) == _abi.KVSEL_E_ARG
    assert _status(lib.kvsel_score_workspace, _score_args(admit=0x5000, tile_mask=0x6000, D=64, **blk),
                   ctypes.byref(nb)) == _abi.KVSEL_E_UNSUPPORTED
    assert _status(lib.kvsel_score_workspace, _score_args(admit=0x5000, tile_mask=0x6000),
                   ctypes.byref(nb)) == _abi.KVSEL_E_ARG          # window mode
    old = _score_args(admit=0x5000, **blk)                            # would be refused if read
    old.struct_size = _abi.ScoreArgs.admit.offset
    assert _status(lib.kvsel_score_workspace, old, ctypes.byref(nb)) == _abi.KVSEL_OK
    old.struct_size = _abi.ScoreArgs.admit.offset - 8
    assert _status(lib.kvsel_score_workspace, old, ctypes.byref(nb)) == _abi.KVSEL_E_ARG


def test_gather_and_redirect_validation_without_device():
    lib = _abi.load()
    a = _abi.GatherArgs()
    a.struct_size = ctypes.sizeof(a)
    a.mode, a.U, a.D, a.dtype, a.bt, a.k = _abi.GATHER_FRESH, 4, 128, _abi.BF16, 32, 16
    a.src_k, a.src_v, a.idx, a.dst_k, a.dst_v, a.src_rows = 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 10
    a.rope, a.theta = 7, 1e6
    nb = ctypes.c_size_t(0)
    assert lib.kvsel_gather_workspace(ctypes.byref(a), ctypes.byref(nb)) == _abi.KVSEL_E_ARG
    a.rope, a.D = _abi.ROPE["raw"], 100
    assert lib.kvsel_gather_workspace(ctypes.byref(a), ctypes.byref(nb)) == _abi.KVSEL_E_UNSUPPORTED
    a.D, a.theta = 128, 0.0
    assert lib.kvsel_gather_workspace(ctypes.byref(a), ctypes.byref(nb)) == _abi.KVSEL_E_ARG
    a.theta = 1e6
    assert lib.kvsel_gather_workspace(ctypes.byref(a), ctypes.byref(nb)) == _abi.KVSEL_OK
    r = _abi.RedirectArgs()
    r.struct_size = ctypes.sizeof(r)
    r.N, r.slot_map, r.keep_mask, r.dead_slot = 10, 0x1000, 0x2000, 5
    r.k_pool, r.v_pool, r.L, r.Hkv, r.D, r.dtype, r.pool_slots = 0x3000, 0x4000, 1, 1, 128, _abi.F32, 6
    assert lib.kvsel_redirect(ctypes.byref(r), None) == _abi.KVSEL_E_UNSUPPORTED
    assert b"fp8" in lib.kvsel_last_error()
    # the kept-index form: no mask and no list is only an empty list (k = 0);
    # a list with k > 0 needs its pointer, and k may not be negative
    r.k_pool = None
    r.keep_mask, r.kept_idx, r.k = None, None, 4
    assert lib.kvsel_redirect(ctypes.byref(r), None) == _abi.KVSEL_E_ARG
    r.k = -1
    r.kept_idx = 0x5000
    assert lib.kvsel_redirect(ctypes.byref(r), None) == _abi.KVSEL_E_ARG
    # a struct that ends before kept_idx (the earlier layout) has the mask form only
    r.struct_size = _abi.RedirectArgs.kept_idx.offset
    r.k = 4
    assert lib.kvsel_redirect(ctypes.byref(r), None) == _abi.KVSEL_E_ARG
    assert b"keep_mask" in lib.kvsel_last_error()
    r.struct_size = _abi.RedirectArgs.kept_idx.offset - 8
    assert lib.kvsel_redirect(ctypes.byref(r), None) == _abi.KVSEL_E_ARG
    assert b"struct_size" in lib.kvsel_last_error()


def test_gather_staging_fields_are_optional_for_the_earlier_layout():
    lib = _abi.load()
    a = _abi.GatherArgs()
    a.mode, a.U, a.D, a.dtype, a.bt, a.k = _abi.GATHER_INCREMENTAL, 4, 128, _abi.BF16, 32, 16
    a.idx, a.prev_idx, a.prev_page, a.pool_k, a.pool_v = 0x3000, 0x4000, 0x5000, 0x6000, 0x7000
    a.page_table, a.n_miss, a.pool_pages, a.rope, a.theta = 0x8000, 0x9000, 20, _abi.ROPE["raw"], 1e6
    nb = ctypes.c_size_t(0)
    call = lambda: lib.kvsel_gather_workspace(ctypes.byref(a), ctypes.byref(nb))
    # staging without a raw source is fine; without either it is not
    a.struct_size = ctypes.sizeof(a)
    a.staged_k, a.staged_v, a.staged_cap = 0xA000, 0xB000, 16
    assert call() == _abi.KVSEL_OK and nb.value == 4 * 16 * 4
    a.staged_v = 0xB008
    assert call() == _abi.KVSEL_E_ARG                 # misaligned staging
    a.staged_k = a.staged_v = None
    assert call() == _abi.KVSEL_E_ARG and b"src" in lib.kvsel_last_error()
    # the earlier layout (ending before staged_k) reads no staging fields
    a.staged_k, a.staged_v = 0xA000, 0xB000
    a.struct_size = _abi.GatherArgs.staged_k.offset
    assert call() == _abi.KVSEL_E_ARG and b"src" in lib.kvsel_last_error()
    a.src_k, a.src_v = 0x1000, 0x2000
    assert call() == _abi.KVSEL_OK
    a.struct_size = _abi.GatherArgs.staged_k.offset - 8
    assert call() == _abi.KVSEL_E_ARG
    # moved hits re-rotated from raw K need that raw source
    a.struct_size = ctypes.sizeof(a)
    a.staged_k, a.staged_v, a.src_k, a.src_v, a.hit_raw = 0xA000, 0xB000, None, None, 1
    assert call() == _abi.KVSEL_E_ARG and b"hit_raw" in lib.kvsel_last_error()
    a.src_k = 0x1000
    assert call() == _abi.KVSEL_OK
    a.hit_raw = 2
    assert call() == _abi.KVSEL_E_ARG


def test_index_validation_without_device():
    lib = _abi.load()
    a = _abi.IndexArgs()
    a.struct_size = ctypes.sizeof(a)
    a.U, a.D, a.dtype, a.bt = 4, 128, _abi.BF16, 32
    a.src_k, a.mu, a.src_unit_stride, a.src_rows = 0x1000, 0x2000, 32 * 64 * 128, 32 * 64
    a.NB, a.b_begin, a.b_count = 64, 0, 64
    call = lambda: lib.kvsel_build_index(ctypes.byref(a), None)
    a.D = 96
    assert call() == _abi.KVSEL_E_UNSUPPORTED
    a.D, a.b_count = 128, 65                      # past NB
    assert call() == _abi.KVSEL_E_ARG
    a.NB, a.b_count = 65, 65                      # past src_rows
    assert call() == _abi.KVSEL_E_ARG and b"src_rows" in lib.kvsel_last_error()
    a.NB, a.b_count, a.bt = 64, 64, 0
    assert call() == _abi.KVSEL_E_ARG
    a.bt, a.mu = 32, 0x2004                       # misaligned output
    assert call() == _abi.KVSEL_E_ARG
    a.mu, a.src_unit_stride = 0x2000, 3           # units not 16-byte aligned
    assert call() == _abi.KVSEL_E_ARG
    a.src_unit_stride, a.b_count = 0, 0           # nothing to do
    assert call() == _abi.KVSEL_OK
    a.struct_size = 8
    assert call() == _abi.KVSEL_E_ARG


def test_free_list_validation_without_device():
    lib = _abi.load()
    a = _abi.FreeListArgs()
    a.struct_size = ctypes.sizeof(a)
    a.N, a.slot_map, a.keep_mask, a.free_slots, a.n_free = 100, 0x1000, 0x2000, 0x3000, 0x4000
    a.dead_slot, a.protected_len, a.n_slots = 50, 0, 64
    nb = ctypes.c_size_t(0)
    assert lib.kvsel_free_list_workspace(ctypes.byref(a), ctypes.byref(nb)) == _abi.KVSEL_OK
    assert nb.value >= 2 * 2 * 4                  # two bitmaps of 64 bits
    assert lib.kvsel_free_list(ctypes.byref(a), None, 0, None) == _abi.KVSEL_E_WORKSPACE
    for field, bad in [("n_slots", 0), ("protected_len", -1), ("N", -5), ("n_free", 0), ("slot_map", 0x1002)]:
        setattr(a, field, bad)
        assert lib.kvsel_free_list_workspace(ctypes.byref(a), ctypes.byref(nb)) == _abi.KVSEL_E_ARG, field
        a.N, a.slot_map, a.n_free, a.n_slots, a.protected_len = 100, 0x1000, 0x4000, 64, 0


def test_compact_validation_without_device():
    lib = _abi.load()
    a = _abi.CompactArgs()
    a.struct_size = ctypes.sizeof(a)
    a.R, a.L, a.Hkv, a.D, a.dtype, a.block_size, a.Y = 2, 3, 8, 128, _abi.BF16, 16, 10
    a.N, a.pool_blocks = 150, 64
    a.keep_mask, a.block_table, a.k_pool, a.v_pool = 0x1000, 0x2000, 0x3000, 0x4000
    a.slot_pos, a.freed_blocks, a.n_freed = 0x5000, 0x6000, 0x7000
    nb = ctypes.c_size_t(0)
    assert lib.kvsel_compact_workspace(ctypes.byref(a), ctypes.byref(nb)) == _abi.KVSEL_OK
    assert nb.value >= 2 * 2 * 160 * 4                 # source and destination lists
    assert lib.kvsel_compact(ctypes.byref(a), None, 0, None) == _abi.KVSEL_E_WORKSPACE
    a.Hkv, a.D = 1, 3                                   # 6-byte slot rows cannot move as 16-byte pieces
    assert lib.kvsel_compact_workspace(ctypes.byref(a), ctypes.byref(nb)) == _abi.KVSEL_E_ARG
    a.Hkv, a.D = 8, 128
    for field, bad in [("N", 161), ("block_size", 0), ("k_pool", 0x3008), ("slot_pos", 0x5002)]:
        good = getattr(a, field)
        setattr(a, field, bad)
        assert lib.kvsel_compact_workspace(ctypes.byref(a), ctypes.byref(nb)) == _abi.KVSEL_E_ARG, field
        setattr(a, field, good)
    a.R = 0
    assert lib.kvsel_compact(ctypes.byref(a), None, 0, None) == _abi.KVSEL_OK


def _decode_args():
    a = _abi.DecodeArgs()
    a.struct_size = ctypes.sizeof(a)
    a.Ra, a.R, a.L, a.Hq, a.Hkv, a.D, a.dtype, a.block_size, a.Y = 4, 8, 2, 32, 8, 128, _abi.BF16, 16, 10
    a.n_cap, a.pool_blocks = 160, 100
    a.q, a.lse, a.k_pool, a.block_table = 0x1000, 0x2000, 0x3000, 0x4000
    a.n_ctx, a.n_seen, a.state = 0x5000, 0x6000, 0x7000
    return a


def test_decode_score_validation_without_device():
    lib = _abi.load()
    for field, bad, want in [("D", 96, _abi.KVSEL_E_UNSUPPORTED), ("dtype", _abi.F32, _abi.KVSEL_E_UNSUPPORTED),
                             ("Hq", 30, _abi.KVSEL_E_ARG), ("Hq", 8 * 17, _abi.KVSEL_E_UNSUPPORTED),
                             ("block_size", 24, _abi.KVSEL_E_UNSUPPORTED), ("q", 0x1008, _abi.KVSEL_E_ARG),
                             ("state", 0, _abi.KVSEL_E_ARG), ("lse", 0x2002, _abi.KVSEL_E_ARG),
                             ("Ra", 9, _abi.KVSEL_E_ARG), ("n_cap", (1 << 30) + 1, _abi.KVSEL_E_ARG),
                             ("scale", float("inf"), _abi.KVSEL_E_ARG), ("Y", 0, _abi.KVSEL_E_ARG)]:
        a = _decode_args()
        setattr(a, field, bad)
        assert lib.kvsel_decode_score(ctypes.byref(a), None) == want, field
    a = _decode_args()
    a.Ra, a.req = 9, 0x8000                             # an explicit request list may exceed R
    a.Hq = 8 * 17
    assert lib.kvsel_decode_score(ctypes.byref(a), None) == _abi.KVSEL_E_UNSUPPORTED
    a = _decode_args()
    a.Ra = 0
    assert lib.kvsel_decode_score(ctypes.byref(a), None) == _abi.KVSEL_OK


def _keep_args():
    a = _abi.KeepScoreArgs()
    a.struct_size = ctypes.sizeof(a)
    a.Rc, a.R, a.L, a.Hkv, a.n_cap = 3, 4, 2, 8, 100
    a.lam, a.top_p = 0.5, 0.9
    a.n_len, a.state, a.keep_score = 0x1000, 0x2000, 0x3000
    return a


def test_keep_score_validation_and_workspace_without_device():
    lib = _abi.load()
    nb = ctypes.c_size_t(0)
    a = _keep_args()
    assert lib.kvsel_keep_score_workspace(ctypes.byref(a), ctypes.byref(nb)) == _abi.KVSEL_OK
    assert nb.value == 3 * 100 * 4                       # scores of the compressing requests
    assert lib.kvsel_keep_score(ctypes.byref(a), None, 0, None) == _abi.KVSEL_E_WORKSPACE
    a.attn_score = 0x4000
    assert lib.kvsel_keep_score_workspace(ctypes.byref(a), ctypes.byref(nb)) == _abi.KVSEL_OK
    assert nb.value == 0
    for field, bad in [("lam", 1.5), ("lam", -0.1), ("top_p", 0.0), ("top_p", 1.01), ("Rc", 5),
                       ("keep_score", 0), ("state", 0x2002), ("L", 0), ("n_cap", -1)]:
        a = _keep_args()
        setattr(a, field, bad)
        assert lib.kvsel_keep_score_workspace(ctypes.byref(a), ctypes.byref(nb)) == _abi.KVSEL_E_ARG, field
    a = _keep_args()
    a.Rc = 0
    assert lib.kvsel_keep_score(ctypes.byref(a), None, 0, None) == _abi.KVSEL_OK


def test_grid_row_limits_are_reported_without_device():
    lib = _abi.load()
    a = _select_args(U=65536)
    nb = ctypes.c_size_t(0)
    assert lib.kvsel_select_workspace(ctypes.byref(a), ctypes.byref(nb)) == _abi.KVSEL_E_UNSUPPORTED
    c = _abi.CompactArgs()
    c.struct_size = ctypes.sizeof(c)
    c.R, c.L, c.Hkv, c.D, c.dtype, c.block_size, c.Y = 65536, 1, 8, 128, _abi.BF16, 16, 1
    c.N, c.pool_blocks = 16, 4
    assert lib.kvsel_compact_workspace(ctypes.byref(c), ctypes.byref(nb)) == _abi.KVSEL_E_UNSUPPORTED


def test_error_messages_are_per_thread():
    import threading
    lib = _abi.load()
    msgs = {}

    def worker(name, budget):
        a = _select_args()
        if budget:
            a.n_sink, a.n_recent = 8, 8                 # 16 forced > k_total 10
        else:
            a.pool, a.pool_k = 1, 4                     # even window
        for _ in range(200):
            lib.kvsel_select(ctypes.byref(a), None, 0, None)
            msgs.setdefault(name, set()).add(lib.kvsel_last_error().decode())

    threads = [threading.Thread(target=worker, args=("b", True)), threading.Thread(target=worker, args=("p", False))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert len(msgs["b"]) == 1 and "k_total" in next(iter(msgs["b"]))
    assert len(msgs["p"]) == 1 and "pool_k" in next(iter(msgs["p"]))
