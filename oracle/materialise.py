"""Materialising a selection: gather with re-RoPE, incremental view update,
slot-map redirect to a dead slot, and the dead-slot attention check.

Test infrastructure only (see ``oracle/__init__``).  Values in float64;
K written to a bfloat16 view is the float64 rotation rounded once
(``numerics.round_to_bf16``); V and unrotated K move bit for bit.
"""
import numpy as np

from .numerics import round_to_bf16, round_to_f16
from .rope import rope_rotate


def gather_view(src_k, src_v, idx, bt, rope="none", theta=1e6, pos0=0,
                style="half", rotary_dim=None, out_round=round_to_bf16):
    """Compact view of one unit.

    KVMem (tiered movement): the selected blocks are packed into contiguous
    logical positions; K is re-rotated for its new position and V is copied
    unchanged.  out[i*bt + o] = src[idx[i]*bt + o] for the i-th kept entry in
    ascending order.  ``rope``: "none" copies K; "raw" rotates raw K to
    p_new = pos0 + i*bt + o; "delta" rotates already-rotated K by
    p_new - p_old with p_old = idx[i]*bt + o.

    src_k, src_v: [NB*bt][D]; idx: [k].  Returns (k_out, v_out) [k*bt][D].
    """
    src_k = np.asarray(src_k, dtype=np.float64)
    src_v = np.asarray(src_v, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    k = idx.shape[0]
    D = src_k.shape[-1]
    rows = (idx[:, None] * bt + np.arange(bt)[None, :]).reshape(-1)      # source rows
    k_out = src_k[rows].copy()
    v_out = src_v[rows].copy()
    p_new = pos0 + np.arange(k * bt)
    if rope == "raw":
        k_out = out_round(rope_rotate(k_out, p_new, theta, style, rotary_dim))
    elif rope == "delta":
        k_out = out_round(rope_rotate(k_out, p_new - rows, theta, style, rotary_dim))
    elif rope != "none":
        raise ValueError(rope)
    assert k_out.shape == (k * bt, D)
    return k_out, v_out


def incremental_view(prev_idx, prev_page, new_idx, pool_k, pool_v, raw_k, raw_v,
                     bt, theta=1e6, pos0=0, style="half", rotary_dim=None,
                     out_round=round_to_bf16, hits="delta"):
    """Update a paged execution view in place from one selection to the next.

    KVMem (tiered movement): pages that overlap across consecutive steps stay
    on the GPU, and missed blocks are scattered in with re-RoPE.  Reading:
    a hit keeps its physical page and V; when its logical position moved its
    K becomes the block's K at the new position, either by rotating the
    page's K in place by (i_new - i_old) * bt (``hits="delta"``: the
    rotation composes, and only the GPU copy is needed) or by rotating the
    block's raw K to pos0 + i_new*bt + o (``hits="raw"``: raw K rotated once,
    so repeated moves do not accumulate bf16 roundings).  The pages of
    blocks that left the view are freed and taken in ascending page order by
    the misses in ascending block order; a miss's K is raw K rotated to
    pos0 + i_new*bt + o and its V is copied.  The new page table lists the
    page of each kept block in chronological order.

    prev_idx, new_idx: [k] ascending block ids; prev_page: [k] page of
    prev_idx[i]; pool_k/pool_v: [P][bt][D]; raw_k/raw_v: [NB][bt][D].
    Returns (pool_k', pool_v', page_table [k], n_miss).
    """
    if hits not in ("delta", "raw"):
        raise ValueError(hits)
    prev_idx = np.asarray(prev_idx, dtype=np.int64)
    prev_page = np.asarray(prev_page, dtype=np.int64)
    new_idx = np.asarray(new_idx, dtype=np.int64)
    pk = np.asarray(pool_k, dtype=np.float64).copy()
    pv = np.asarray(pool_v, dtype=np.float64).copy()
    raw_k = np.asarray(raw_k, dtype=np.float64)
    raw_v = np.asarray(raw_v, dtype=np.float64)
    where_prev = {int(b): i for i, b in enumerate(prev_idx)}
    new_set = set(int(b) for b in new_idx)
    freed = sorted(int(prev_page[i]) for i, b in enumerate(prev_idx) if int(b) not in new_set)
    page_table = np.empty(new_idx.shape[0], dtype=np.int64)
    o = np.arange(bt)
    n_miss = 0
    for i_new, b in enumerate(new_idx):
        b = int(b)
        if b in where_prev:
            i_old = where_prev[b]
            page = int(prev_page[i_old])
            delta = (i_new - i_old) * bt
            if delta != 0 and hits == "delta":
                pk[page] = out_round(rope_rotate(pk[page], np.full(bt, delta), theta,
                                                 style, rotary_dim))
            elif delta != 0:
                pk[page] = out_round(rope_rotate(raw_k[b], pos0 + i_new * bt + o, theta,
                                                 style, rotary_dim))
        else:
            page = freed[n_miss]
            n_miss += 1
            pk[page] = out_round(rope_rotate(raw_k[b], pos0 + i_new * bt + o, theta,
                                             style, rotary_dim))
            pv[page] = raw_v[b]
        page_table[i_new] = page
    return pk, pv, page_table, n_miss


def redirect(slot_map, keep_mask, dead_slot):
    """Slot-map redirect (IntentKV §4, redirect; §2 Q2 layout).

    Every dropped logical position points at the dead slot; kept positions and
    their physical slots are untouched.  Positions already dead stay dead.
    """
    sm = np.asarray(slot_map, dtype=np.int64)
    return np.where(np.asarray(keep_mask, dtype=bool), sm, dead_slot)


def free_list(slot_map, keep_mask, dead_slot, protected_len=0):
    """Physical slots a compression step may return to the allocator
    (IntentKV §7, alias-aware deallocation; §4 minimum check 6).

    A dropped logical position j (keep_mask[j] false) frees its slot
    u = slot_map[j] only if (a) j is outside the radix-protected prefix
    (j >= protected_len), (b) u is not the dead slot, and (c) no kept
    position maps to u.  slot_map is the map before the redirect.  Returns
    the distinct freed slots in ascending order (int64).
    """
    sm = np.asarray(slot_map, dtype=np.int64)
    keep = np.asarray(keep_mask, dtype=bool)
    kept_slots = set(int(u) for u in sm[keep])
    freed = set()
    for j in range(sm.shape[0]):
        u = int(sm[j])
        if keep[j] or j < protected_len or u == dead_slot or u in kept_slots:
            continue
        freed.add(u)
    return np.array(sorted(freed), dtype=np.int64)


def tail_compact(keep_mask, block_table, block_size, k_pool, v_pool):
    """In-place compaction of one request's paged KV into its tail blocks
    (ActKV §7.2, conflict-free slot planning; Algorithm 4).

    The request holds Y logical blocks (block_table[y] is the physical block
    of logical block y) and N = len(keep_mask) <= Y * block_size positions.
    With K kept positions, the target region is the last X = ceil(K / bs)
    logical blocks, starting at slot t0 = (Y - X) * bs.  Sources are the kept
    positions before t0, destinations the slots from t0 on that hold no kept
    entry (dropped positions, or empty slots past N), both in ascending order;
    the i-th source moves to the i-th destination.  Sources and destinations
    are disjoint, so one pass of copies suffices.

    k_pool, v_pool: [pool_blocks][bs][...] arrays, not modified.  Returns
    (k_pool', v_pool', slot_pos, freed): the pools after the copies;
    slot_pos [Y * bs] = the original logical position each slot holds
    afterwards (-1 for empty slots and for the freed blocks); freed = the
    physical blocks of logical blocks [0, Y - X), in order.
    """
    keep = np.asarray(keep_mask, dtype=bool)
    bt = np.asarray(block_table, dtype=np.int64)
    bs = int(block_size)
    Y, N = bt.shape[0], keep.shape[0]
    assert N <= Y * bs
    n_kept = int(keep.sum())
    X = -(-n_kept // bs)
    t0 = (Y - X) * bs
    kept_slot = np.zeros(Y * bs, dtype=bool)
    kept_slot[:N] = keep
    sources = [p for p in range(min(t0, N)) if keep[p]]
    dests = [s for s in range(t0, Y * bs) if not kept_slot[s]]
    assert len(dests) >= len(sources)
    kp, vp = np.array(k_pool, copy=True), np.array(v_pool, copy=True)

    def phys(s):
        return bt[s // bs], s % bs

    slot_pos = np.full(Y * bs, -1, dtype=np.int64)
    for s in range(t0, Y * bs):
        if kept_slot[s]:
            slot_pos[s] = s
    for src, dst in zip(sources, dests):
        (bs_, os_), (bd, od) = phys(src), phys(dst)
        kp[bd, od] = k_pool[bs_, os_]
        vp[bd, od] = v_pool[bs_, os_]
        slot_pos[dst] = src
    return kp, vp, slot_pos, bt[: Y - X].copy()


def sentinel_rows(dtype, D):
    """K and V rows of the dead slot (IntentKV §2 Q2): K = -1e4, V = 0,
    each rounded once to the pool's storage format ("bf16" or "f16")."""
    rnd = {"bf16": round_to_bf16, "f16": round_to_f16}[dtype]
    return rnd(np.full(D, -1.0e4)), np.zeros(D)


def decode_attention_slots(q, pool_k, pool_v, slot_map, scale=None):
    """Decode attention through a slot map over all N logical positions.

    ActKV §2 (attention output): o = sum_j softmax_j(q . K[s_j] / sqrt(D)) V[s_j].
    q: [D]; pool_k/pool_v: [n_slots][D]; slot_map: [N].
    """
    q = np.asarray(q, dtype=np.float64)
    sm = np.asarray(slot_map, dtype=np.int64)
    K = np.asarray(pool_k, dtype=np.float64)[sm]
    V = np.asarray(pool_v, dtype=np.float64)[sm]
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[0])
    s = (K @ q) * scale
    m = np.max(s)
    w = np.exp(s - m)
    # sequential sums in position order: an exactly-zero weight adds nothing
    num = np.zeros(V.shape[1])
    den = 0.0
    for j in range(w.shape[0]):
        num = num + w[j] * V[j]
        den = den + w[j]
    return num / den


def decode_attention_hard(q, pool_k, pool_v, slot_map, keep_mask, scale=None):
    """The same attention restricted to the kept positions (a hard mask)."""
    keep = np.asarray(keep_mask, dtype=bool)
    return decode_attention_slots(q, pool_k, pool_v, np.asarray(slot_map)[keep], scale)
