"""Python binding of libkvsel: argument marshalling only.

Each function checks the torch tensors it is handed (device, dtype,
contiguity), fills the C args struct with their data pointers, sizes and
allocates the workspace the library asks for (torch owns device memory), and
calls the C entry point of the same name on the current torch stream.  All
computation runs in the library's HIP kernels; a non-OK status raises
``KvselError`` with the library's message.
"""
import ctypes

import torch

from . import _abi

_DT = {torch.float32: _abi.F32, torch.bfloat16: _abi.BF16, torch.float16: _abi.F16}


class KvselError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (_abi.STATUS_NAMES.get(status, status), msg))
        self.status = status


def _check(status):
    if status != _abi.KVSEL_OK:
        raise KvselError(status, _abi.load().kvsel_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _want(t, name, dtype=None, shape=None, numel=None):
    """Check a tensor the C call will address through a raw pointer: its
    dtype, its exact shape, or at least `numel` elements.  A wrong size would
    let a kernel read or write past the buffer, so it is refused here."""
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if numel is not None and t.numel() < numel:
        raise ValueError("%s needs at least %d elements, has %d" % (name, numel, t.numel()))
    return t


def _wptr(t, name, dtype=None, shape=None, numel=None):
    """_want, then the tensor's device pointer."""
    return _ptr(_want(t, name, dtype, shape, numel))


def _dtype(t):
    if t.dtype not in _DT:
        raise ValueError("unsupported dtype %s" % t.dtype)
    return _DT[t.dtype]


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(nbytes, device, workspace):
    """The caller's workspace as it is (the library checks its size: a
    memory-mode score runs in more passes on a shorter one, other calls
    report KVSEL_E_WORKSPACE), or a new one of the size the query returned."""
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        _want(workspace, "workspace", torch.uint8)
        return workspace, workspace.numel()
    w = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return w, nbytes


def version():
    return int(_abi.load().kvsel_version())


# ------------------------------------------------------------------ score

def _score_call(a, device, workspace, stream):
    lib = _abi.load()
    nb = ctypes.c_size_t(0)
    _check(lib.kvsel_score_workspace(ctypes.byref(a), ctypes.byref(nb)))
    ws, wsz = _workspace(nb.value, device, workspace)
    _check(lib.kvsel_score(ctypes.byref(a), _ptr(ws), wsz, _stream(stream)))
    return ws


def score_window(q, k, out, *, causal=True, lse_in=None, lse_out=None, head_agg="sum",
                 row_agg="sum", pool="none", pool_k=1, scale=0.0, workspace=None, stream=None):
    """kvsel_score, window mode.  q [L][Hq][W][D], k [L][Hkv][N][D] (one dtype),
    out [L*Hkv][N] float32 (or None to compute only lse_out); lse_in/lse_out
    [L][Hq][W] float32 (optional)."""
    L, Hq, W, D = q.shape
    _, Hkv, N, _ = k.shape
    a = _abi.ScoreArgs()
    a.struct_size = ctypes.sizeof(_abi.ScoreArgs)
    a.mode = _abi.SCORE_WINDOW
    a.q_dtype, a.k_dtype = _dtype(q), _dtype(k)
    a.L, a.Hq, a.Hkv, a.D, a.W, a.S, a.N = L, Hq, Hkv, D, W, 1, N
    a.q, a.k = _ptr(q), _ptr(k)
    a.causal = 1 if causal else 0
    a.lse_in = _wptr(lse_in, "lse_in", torch.float32, (L, Hq, W))
    a.lse_out = _wptr(lse_out, "lse_out", torch.float32, (L, Hq, W))
    a.head_agg, a.row_agg = _abi.AGG[head_agg], _abi.AGG[row_agg]
    a.pool, a.pool_k = _abi.POOL[pool], pool_k
    a.scale = scale
    a.scores = _wptr(out, "out", torch.float32, numel=L * Hkv * N)   # None with lse_out: LSE only
    return _score_call(a, q.device, workspace, stream)


def score_memory(m, k_pool, page_table, n, out, *, page_size, slot_map=None, dead_slot=0, n_sink=0,
                 n_recent=0, reduce="global", pool="none", pool_k=1, scale=0.0, workspace=None,
                 stream=None):
    """kvsel_score, memory mode.  m [L][Hq][D] float32; k_pool
    [L][pool_pages][page_size][Hkv][D]; page_table int32; out [N] (global)
    or [L*Hkv][N] (per_unit) float32."""
    L, Hq, D = m.shape
    _, P, ps, Hkv, _ = k_pool.shape
    assert ps == page_size
    a = _abi.ScoreArgs()
    a.struct_size = ctypes.sizeof(_abi.ScoreArgs)
    a.mode = _abi.SCORE_MEMORY
    a.q_dtype, a.k_dtype = _dtype(m), _dtype(k_pool)
    a.L, a.Hq, a.Hkv, a.D, a.W, a.S, a.N = L, Hq, Hkv, D, 1, 1, n
    a.q, a.k = _wptr(m, "m", torch.float32), _ptr(k_pool)
    a.page_table = _wptr(page_table, "page_table", torch.int32, numel=-(-n // page_size))
    a.page_size, a.pool_pages = page_size, P
    a.slot_map, a.dead_slot = _wptr(slot_map, "slot_map", torch.int32, numel=n), dead_slot
    a.n_sink, a.n_recent = n_sink, n_recent
    a.reduce = _abi.REDUCE[reduce]
    a.pool, a.pool_k = _abi.POOL[pool], pool_k
    a.scale = scale
    a.scores = _wptr(out, "out", torch.float32, numel=n if reduce == "global" else L * Hkv * n)
    return _score_call(a, m.device, workspace, stream)


def score_block(q, mu, out, *, n_kv_heads, n_begin=0, n_count=None, qbar=None, qbar_valid=False,
                scale=0.0, admit=None, tile_mask=None, workspace=None, stream=None):
    """kvsel_score, block mode.  q [S][L][Hq][W][D] (or None with a valid qbar),
    mu [L][Hkv][NB][D] float16, out [S][L*Hkv][n_count] float32,
    qbar [S][L][Hkv][D] float32 (optional).  With admit ([S][L*Hkv] float32,
    from a tiled select) and tile_mask ([S][L*Hkv][ceil(n_count/64)] int64,
    the uint64 mask words) the output is the packed tile form."""
    L, Hkv, NB, D = mu.shape
    assert Hkv == n_kv_heads
    if n_count is None:
        n_count = NB - n_begin
    a = _abi.ScoreArgs()
    a.struct_size = ctypes.sizeof(_abi.ScoreArgs)
    a.mode = _abi.SCORE_BLOCK
    if q is not None:
        S, _, Hq, W, _ = q.shape
        a.q_dtype = _dtype(q)
    else:
        S, Hq, W = qbar.shape[0], n_kv_heads, 1
        a.q_dtype = _abi.F32
    a.k_dtype = _dtype(mu)
    a.L, a.Hq, a.Hkv, a.D, a.W, a.S, a.N = L, Hq, Hkv, D, W, S, NB
    a.q, a.k = _ptr(q), _wptr(mu, "mu", torch.float16)
    a.n_begin, a.n_count = n_begin, n_count
    a.qbar, a.qbar_valid = _wptr(qbar, "qbar", torch.float32, (S, L, Hkv, D)), 1 if qbar_valid else 0
    a.scale = scale
    a.scores = _wptr(out, "out", torch.float32, numel=S * L * Hkv * n_count)
    a.admit = _wptr(admit, "admit", torch.float32, numel=S * L * Hkv)
    a.tile_mask = _wptr(tile_mask, "tile_mask", torch.int64, numel=S * L * Hkv * ((n_count + 63) // 64))
    return _score_call(a, mu.device, workspace, stream)


# ------------------------------------------------------------------ select

def _select_args(scores, kept_idx, *, k_total, n_sink, n_recent, n_total, base, keep_mask, n_kept, slot_map,
                 dead_slot, cand_score, cand_idx, cand_count, finalize, pool, pool_k, tile_mask=None, admit=None):
    U, n = scores.shape
    if n_total is None:
        n_total = base + n
    if scores.stride(1) != 1:
        raise ValueError("score rows must be contiguous")
    if scores.dtype != torch.float32:
        raise TypeError("scores must be float32")
    a = _abi.SelectArgs()
    a.struct_size = ctypes.sizeof(_abi.SelectArgs)
    a.U, a.n, a.row_stride = U, n, scores.stride(0)
    a.scores = scores.data_ptr() if scores.is_cuda else None
    a.base, a.n_total = base, n_total
    a.k_total, a.n_sink, a.n_recent = k_total, n_sink, n_recent
    for t, name, dt, numel in ((slot_map, "slot_map", torch.int32, n_total),
                               (cand_score, "cand_score", torch.float32, U * k_total),
                               (cand_idx, "cand_idx", torch.int32, U * k_total), (cand_count, "cand_count", torch.int32, U),
                               (kept_idx, "kept_idx", torch.int32, U * k_total),
                               (keep_mask, "keep_mask", torch.uint8, U * n_total), (n_kept, "n_kept", torch.int32, U)):
        _want(t, name, dt, numel=numel)
    a.slot_map, a.dead_slot = _ptr(slot_map), dead_slot
    a.cand_score, a.cand_idx, a.cand_count = _ptr(cand_score), _ptr(cand_idx), _ptr(cand_count)
    a.finalize = 1 if finalize else 0
    a.kept_idx, a.keep_mask, a.n_kept = _ptr(kept_idx), _ptr(keep_mask), _ptr(n_kept)
    a.pool, a.pool_k = _abi.POOL[pool], pool_k
    a.tile_mask = _wptr(tile_mask, "tile_mask", torch.int64, numel=U * ((n + 63) // 64))
    a.admit = _wptr(admit, "admit", torch.float32, numel=U)
    return a


def select(scores, kept_idx, *, k_total, n_sink, n_recent, n_total=None, base=0, keep_mask=None,
           n_kept=None, slot_map=None, dead_slot=0, cand_score=None, cand_idx=None, cand_count=None,
           finalize=True, pool="none", pool_k=1, tile_mask=None, admit=None, workspace=None, stream=None):
    """kvsel_select.  scores [U][n] float32 (rows may be a strided view of
    contiguous memory: pass the 2-D tensor); kept_idx [U][k_total] int32.
    pool/pool_k rank pooled scores (untiled calls).  Tiled calls: tile_mask
    ([U][ceil(n/64)] int64) marks a packed tile; admit ([U] float32)
    receives the admission threshold for the next tile.  Returns the
    workspace (untiled calls need one; pass it back to reuse it)."""
    a = _select_args(scores, kept_idx, k_total=k_total, n_sink=n_sink, n_recent=n_recent, n_total=n_total,
                     base=base, keep_mask=keep_mask, n_kept=n_kept, slot_map=slot_map, dead_slot=dead_slot,
                     cand_score=cand_score, cand_idx=cand_idx, cand_count=cand_count, finalize=finalize,
                     pool=pool, pool_k=pool_k, tile_mask=tile_mask, admit=admit)
    lib = _abi.load()
    nb = ctypes.c_size_t(0)
    _check(lib.kvsel_select_workspace(ctypes.byref(a), ctypes.byref(nb)))
    ws, wsz = _workspace(nb.value, scores.device, workspace)
    _check(lib.kvsel_select(ctypes.byref(a), _ptr(ws), wsz, _stream(stream)))
    return ws


def select_noalloc(scores, kept_idx, *, k_total, n_sink, n_recent, n_total=None, base=0, keep_mask=None,
                   n_kept=None, slot_map=None, dead_slot=0, cand_score=None, cand_idx=None, cand_count=None,
                   finalize=True, pool="none", pool_k=1, tile_mask=None, admit=None, stream=None):
    """kvsel_select_noalloc: kvsel_select with its scratch in the library's
    fixed per-device array (nothing is allocated, here or in the library).
    Calls that overlap on one GPU share that array and race."""
    a = _select_args(scores, kept_idx, k_total=k_total, n_sink=n_sink, n_recent=n_recent, n_total=n_total,
                     base=base, keep_mask=keep_mask, n_kept=n_kept, slot_map=slot_map, dead_slot=dead_slot,
                     cand_score=cand_score, cand_idx=cand_idx, cand_count=cand_count, finalize=finalize,
                     pool=pool, pool_k=pool_k, tile_mask=tile_mask, admit=admit)
    _check(_abi.load().kvsel_select_noalloc(ctypes.byref(a), _stream(stream)))


# ------------------------------------------------------------------ gather

def _gather_args(src_k, src_v, idx, *, bt, D, src_rows, src_offsets, src_unit_stride, rope, theta,
                 pos0, style, rotary_dim, dtype_of=None):
    a = _abi.GatherArgs()
    a.struct_size = ctypes.sizeof(_abi.GatherArgs)
    a.U, a.k = idx.shape
    a.D, a.dtype, a.bt = D, _dtype(src_k if dtype_of is None else dtype_of), bt
    a.src_k, a.src_v = _ptr(src_k), _ptr(src_v)
    a.src_offsets = _wptr(src_offsets, "src_offsets", torch.int64, numel=a.U)
    a.src_unit_stride, a.src_rows = src_unit_stride, src_rows
    a.idx = _wptr(idx, "idx", torch.int32)
    a.rope, a.style, a.rotary_dim = _abi.ROPE[rope], _abi.STYLE[style], rotary_dim
    a.theta, a.pos0 = theta, pos0
    return a


def gather_rerope(src_k, src_v, idx, dst_k, dst_v, *, bt, D, src_rows, src_offsets=None,
                  src_unit_stride=0, n_idx=None, rope="none", theta=1e6, pos0=0, style="half",
                  rotary_dim=0, stream=None):
    """kvsel_gather_rerope, FRESH mode.  idx [U][k] int32; dst [U][k*bt][D]."""
    a = _gather_args(src_k, src_v, idx, bt=bt, D=D, src_rows=src_rows, src_offsets=src_offsets,
                     src_unit_stride=src_unit_stride, rope=rope, theta=theta, pos0=pos0, style=style,
                     rotary_dim=rotary_dim)
    a.mode = _abi.GATHER_FRESH
    a.n_idx = _wptr(n_idx, "n_idx", torch.int32, numel=a.U)
    rows = a.U * a.k * bt * D
    a.dst_k = _wptr(dst_k, "dst_k", src_k.dtype, numel=rows)
    a.dst_v = _wptr(dst_v, "dst_v", src_v.dtype, numel=rows)
    lib = _abi.load()
    _check(lib.kvsel_gather_rerope(ctypes.byref(a), None, 0, _stream(stream)))


def gather_incremental(src_k, src_v, idx, prev_idx, prev_page, pool_k, pool_v, page_table, n_miss, *,
                       bt, D, src_rows=0, src_offsets=None, src_unit_stride=0, rope="raw", theta=1e6,
                       pos0=0, style="half", rotary_dim=0, staged_k=None, staged_v=None, hit_raw=False,
                       workspace=None, stream=None):
    """kvsel_gather_rerope, INCREMENTAL mode.  pool_k/pool_v
    [U][pool_pages][bt][D] updated in place; page_table [U][k], n_miss [U] out.
    Misses come from src (by block id) or, with staged_k/staged_v
    [U][staged_cap][bt][D], from packed staging (the i-th miss of a unit at
    entry i); src_k/src_v may then be None.  hit_raw re-rotates moved hits
    from src_k at their new position instead of rotating the page in place."""
    a = _gather_args(src_k, src_v, idx, bt=bt, D=D, src_rows=src_rows, src_offsets=src_offsets,
                     src_unit_stride=src_unit_stride, rope=rope, theta=theta, pos0=pos0, style=style,
                     rotary_dim=rotary_dim, dtype_of=pool_k)
    a.mode = _abi.GATHER_INCREMENTAL
    if staged_k is not None:
        cap = staged_k.shape[1]
        _want(staged_k, "staged_k", pool_k.dtype, (a.U, cap, bt, D))
        _want(staged_v, "staged_v", pool_k.dtype, (a.U, cap, bt, D))
        a.staged_k, a.staged_v, a.staged_cap = _ptr(staged_k), _ptr(staged_v), cap
    a.hit_raw = 1 if hit_raw else 0
    a.prev_idx = _wptr(prev_idx, "prev_idx", torch.int32, numel=a.U * a.k)
    a.prev_page = _wptr(prev_page, "prev_page", torch.int32, numel=a.U * a.k)
    a.pool_k, a.pool_v, a.pool_pages = _ptr(pool_k), _ptr(pool_v), pool_k.shape[1]
    a.page_table = _wptr(page_table, "page_table", torch.int32, numel=a.U * a.k)
    a.n_miss = _wptr(n_miss, "n_miss", torch.int32, numel=a.U)
    lib = _abi.load()
    nb = ctypes.c_size_t(0)
    _check(lib.kvsel_gather_workspace(ctypes.byref(a), ctypes.byref(nb)))
    ws, wsz = _workspace(nb.value, pool_k.device, workspace)
    _check(lib.kvsel_gather_rerope(ctypes.byref(a), _ptr(ws), wsz, _stream(stream)))
    return ws


# ------------------------------------------------------------------ redirect / memory

def redirect(slot_map, keep_mask, dead_slot, *, kept_idx=None, k_pool=None, v_pool=None, stream=None):
    """kvsel_redirect.  slot_map [N] int32 (in place); the kept set as
    keep_mask [N] uint8, or (keep_mask None) as kept_idx [k] int32, ascending
    with a -1 tail allowed.  With k_pool/v_pool ([L][pool_slots][Hkv][D]
    views of the paged pools) the dead slot's sentinel rows are written first."""
    a = _abi.RedirectArgs()
    a.struct_size = ctypes.sizeof(_abi.RedirectArgs)
    a.N = slot_map.numel()
    a.slot_map = _wptr(slot_map, "slot_map", torch.int32)
    a.keep_mask = _wptr(keep_mask, "keep_mask", torch.uint8, numel=a.N)
    if keep_mask is None and kept_idx is None:
        raise ValueError("give keep_mask or kept_idx")
    if keep_mask is None:
        a.kept_idx = _wptr(kept_idx.reshape(-1), "kept_idx", torch.int32)
        a.k = kept_idx.numel()
    a.dead_slot = dead_slot
    if k_pool is not None:
        L, slots, Hkv, D = k_pool.shape
        a.k_pool, a.v_pool = _ptr(k_pool), _ptr(v_pool)
        a.L, a.Hkv, a.D, a.dtype, a.pool_slots = L, Hkv, D, _dtype(k_pool), slots
    lib = _abi.load()
    _check(lib.kvsel_redirect(ctypes.byref(a), _stream(stream)))


def memory_update(q_turn, m, *, decay=0.9, stream=None):
    """kvsel_memory_update.  q_turn [L][Hq][W][D]; m [L][Hq][D] float32 in place."""
    L, Hq, W, D = q_turn.shape
    a = _abi.MemUpdArgs()
    a.struct_size = ctypes.sizeof(_abi.MemUpdArgs)
    a.L, a.Hq, a.D, a.W = L, Hq, D, W
    a.q_dtype = _dtype(q_turn)
    a.q_turn, a.M, a.decay = _ptr(q_turn), _wptr(m, "m", torch.float32, (L, Hq, D)), decay
    lib = _abi.load()
    _check(lib.kvsel_memory_update(ctypes.byref(a), _stream(stream)))


def build_index(raw_k, mu, *, bt, D, src_rows, NB=None, b_begin=0, b_count=None, src_offsets=None,
                src_unit_stride=0, stream=None):
    """kvsel_build_index.  raw_k: the raw-key store (any shape; unit u starts
    at element src_offsets[u], or u * src_unit_stride); mu: float16 [U][NB][D],
    written for blocks [b_begin, b_begin + b_count) of every unit."""
    if mu.dtype != torch.float16:
        raise TypeError("mu must be float16")
    U = mu.shape[0]
    NB = mu.shape[1] if NB is None else NB
    b_count = NB - b_begin if b_count is None else b_count
    a = _abi.IndexArgs()
    a.struct_size = ctypes.sizeof(_abi.IndexArgs)
    a.U, a.D, a.dtype, a.bt = U, D, _dtype(raw_k), bt
    a.src_k, a.src_unit_stride, a.src_rows = _ptr(raw_k), src_unit_stride, src_rows
    a.src_offsets = _wptr(src_offsets, "src_offsets", torch.int64, numel=U)
    a.NB, a.b_begin, a.b_count, a.mu = NB, b_begin, b_count, _ptr(mu)
    lib = _abi.load()
    _check(lib.kvsel_build_index(ctypes.byref(a), _stream(stream)))


def free_list(slot_map, keep_mask, dead_slot, free_slots, n_free, *, n_slots, protected_len=0, workspace=None,
              stream=None):
    """kvsel_free_list.  slot_map [N] int32 (before the redirect); keep_mask [N]
    uint8; free_slots [N] int32 and n_free [1] int32 are written.  Returns the
    workspace it used."""
    N = slot_map.shape[0]
    a = _abi.FreeListArgs()
    a.struct_size = ctypes.sizeof(_abi.FreeListArgs)
    for t, name, dt, numel in ((slot_map, "slot_map", torch.int32, None), (keep_mask, "keep_mask", torch.uint8, N),
                               (free_slots, "free_slots", torch.int32, N), (n_free, "n_free", torch.int32, 1)):
        _want(t, name, dt, numel=numel)
    a.N, a.slot_map, a.keep_mask, a.dead_slot = N, _ptr(slot_map), _ptr(keep_mask), dead_slot
    a.protected_len, a.n_slots, a.free_slots, a.n_free = protected_len, n_slots, _ptr(free_slots), _ptr(n_free)
    lib = _abi.load()
    nb = ctypes.c_size_t(0)
    _check(lib.kvsel_free_list_workspace(ctypes.byref(a), ctypes.byref(nb)))
    ws, wsz = _workspace(nb.value, slot_map.device, workspace)
    _check(lib.kvsel_free_list(ctypes.byref(a), _ptr(ws), wsz, _stream(stream)))
    return ws


def compact(keep_mask, block_table, k_pool, v_pool, slot_pos, freed_blocks, n_freed, *, block_size,
            workspace=None, stream=None):
    """kvsel_compact.  keep_mask [R][N] uint8; block_table [R][Y] int32;
    k_pool, v_pool [L][pool_blocks][block_size][Hkv][D] (in place); slot_pos
    [R][Y*block_size], freed_blocks [R][Y], n_freed [R] int32 are written.
    Returns the workspace it used."""
    R, N = keep_mask.shape
    Y = block_table.shape[1]
    L, P, bs, Hkv, D = k_pool.shape
    if bs != block_size:
        raise ValueError("k_pool's block dimension must equal block_size")
    a = _abi.CompactArgs()
    a.struct_size = ctypes.sizeof(_abi.CompactArgs)
    a.R, a.L, a.Hkv, a.D, a.dtype, a.block_size, a.Y = R, L, Hkv, D, _dtype(k_pool), block_size, Y
    a.N, a.pool_blocks = N, P
    for t, name, dt, shape, numel in ((keep_mask, "keep_mask", torch.uint8, None, None),
                                      (block_table, "block_table", torch.int32, (R, Y), None),
                                      (v_pool, "v_pool", k_pool.dtype, tuple(k_pool.shape), None),
                                      (slot_pos, "slot_pos", torch.int32, (R, Y * block_size), None),
                                      (freed_blocks, "freed_blocks", torch.int32, (R, Y), None),
                                      (n_freed, "n_freed", torch.int32, None, R)):
        _want(t, name, dt, shape, numel)
    a.keep_mask, a.block_table, a.k_pool, a.v_pool = _ptr(keep_mask), _ptr(block_table), _ptr(k_pool), _ptr(v_pool)
    a.slot_pos, a.freed_blocks, a.n_freed = _ptr(slot_pos), _ptr(freed_blocks), _ptr(n_freed)
    lib = _abi.load()
    nb = ctypes.c_size_t(0)
    _check(lib.kvsel_compact_workspace(ctypes.byref(a), ctypes.byref(nb)))
    ws, wsz = _workspace(nb.value, k_pool.device, workspace)
    _check(lib.kvsel_compact(ctypes.byref(a), _ptr(ws), wsz, _stream(stream)))
    return ws


def decode_score(q, lse, k_pool, block_table, n_ctx, n_seen, state, *, req=None, scale=0.0, stream=None):
    """kvsel_decode_score.  q [L][Ra][Hq][D] (bf16/f16, post-RoPE); lse
    [L][Ra][Hq] float32 (natural log); k_pool [L][pool_blocks][block_size][Hkv][D];
    block_table [R][Y], n_ctx [R], n_seen [R] int32; state [L][R][Hkv][n_cap]
    float32, updated in place; req [Ra] int32 or None (rows 0..Ra-1)."""
    L, Ra, Hq, D = q.shape
    _, P, bs, Hkv, _ = k_pool.shape
    R, Y = block_table.shape
    if state.shape[:3] != (L, R, Hkv):
        raise ValueError("state must be [L][R][Hkv][n_cap]")
    if q.dtype != k_pool.dtype:
        raise ValueError("q and k_pool must share a dtype")
    a = _abi.DecodeArgs()
    a.struct_size = ctypes.sizeof(_abi.DecodeArgs)
    a.Ra, a.R, a.L, a.Hq, a.Hkv, a.D = Ra, R, L, Hq, Hkv, D
    a.dtype, a.block_size, a.Y, a.scale = _dtype(k_pool), bs, Y, scale
    a.n_cap, a.pool_blocks = state.shape[3], P
    for t, name, dt, shape, numel in ((req, "req", torch.int32, (Ra,), None),
                                      (lse, "lse", torch.float32, (L, Ra, Hq), None),
                                      (block_table, "block_table", torch.int32, None, None),
                                      (n_ctx, "n_ctx", torch.int32, None, R), (n_seen, "n_seen", torch.int32, None, R),
                                      (state, "state", torch.float32, None, None)):
        _want(t, name, dt, shape, numel)
    a.req, a.q, a.lse, a.k_pool = _ptr(req), _ptr(q), _ptr(lse), _ptr(k_pool)
    a.block_table, a.n_ctx, a.n_seen, a.state = _ptr(block_table), _ptr(n_ctx), _ptr(n_seen), _ptr(state)
    _check(_abi.load().kvsel_decode_score(ctypes.byref(a), _stream(stream)))


def keep_score(state, keep, n_len, *, lam, top_p=0.9, req=None, attn_score=None, hit=None, workspace=None,
               stream=None):
    """kvsel_keep_score.  state [L][R][Hkv][n_cap] float32 running means;
    keep [R][n_cap] float32 keep scores, updated in place; n_len [R] int32;
    req [Rc] int32 or None (all R); attn_score [R][n_cap] float32 and hit
    [R][n_cap] uint8 optional outputs.  Returns the workspace it used."""
    L, R, Hkv, n_cap = state.shape
    Rc = R if req is None else req.shape[0]
    a = _abi.KeepScoreArgs()
    a.struct_size = ctypes.sizeof(_abi.KeepScoreArgs)
    a.Rc, a.R, a.L, a.Hkv, a.reserved, a.n_cap = Rc, R, L, Hkv, 0, n_cap
    a.lam, a.top_p = lam, top_p
    for t, name, dt, shape, numel in ((req, "req", torch.int32, (Rc,), None), (n_len, "n_len", torch.int32, None, R),
                                      (state, "state", torch.float32, None, None),
                                      (keep, "keep", torch.float32, (R, n_cap), None),
                                      (attn_score, "attn_score", torch.float32, (R, n_cap), None),
                                      (hit, "hit", torch.uint8, (R, n_cap), None)):
        _want(t, name, dt, shape, numel)
    a.req, a.n_len, a.state, a.keep_score = _ptr(req), _ptr(n_len), _ptr(state), _ptr(keep)
    a.attn_score, a.hit = _ptr(attn_score), _ptr(hit)
    lib = _abi.load()
    nb = ctypes.c_size_t(0)
    _check(lib.kvsel_keep_score_workspace(ctypes.byref(a), ctypes.byref(nb)))
    ws, wsz = _workspace(nb.value, state.device, workspace)
    _check(lib.kvsel_keep_score(ctypes.byref(a), _ptr(ws), wsz, _stream(stream)))
    return ws
