"""Pins for RoPE, gather, incremental view update, redirect and the dead-slot
mask (CPU only)."""
import math

import numpy as np
import pytest

from oracle import materialise as om
from oracle import numerics
from oracle.rope import inv_freq, rope_rotate
from parity import bf16_ulp, pair_norm


# ---------------------------------------------------------------- RoPE

def test_rope_d2_theta1_is_rotation_by_p_radians():
    for p in [0, 1, 2, 7, 100, 12345]:
        y = rope_rotate(np.array([1.0, 0.0]), p, theta=1.0)
        np.testing.assert_allclose(y, [math.cos(p), math.sin(p)], atol=1e-12)
        y = rope_rotate(np.array([0.0, 1.0]), p, theta=1.0)
        np.testing.assert_allclose(y, [-math.sin(p), math.cos(p)], atol=1e-12)


def test_rope_pairs_and_frequencies_d4():
    # theta = 100, D = 4: inv_freq = (1, 0.1); rotate-half pairs (0,2) and (1,3)
    np.testing.assert_allclose(inv_freq(4, 100.0), [1.0, 0.1], rtol=1e-15)
    x = np.array([1.0, 2.0, 3.0, 4.0])
    p = 3
    c0, s0, c1, s1 = math.cos(3), math.sin(3), math.cos(0.3), math.sin(0.3)
    want = [1 * c0 - 3 * s0, 2 * c1 - 4 * s1, 1 * s0 + 3 * c0, 2 * s1 + 4 * c1]
    np.testing.assert_allclose(rope_rotate(x, p, 100.0), want, atol=1e-12)
    want_il = [1 * c0 - 2 * s0, 1 * s0 + 2 * c0, 3 * c1 - 4 * s1, 3 * s1 + 4 * c1]
    np.testing.assert_allclose(rope_rotate(x, p, 100.0, style="interleaved"), want_il, atol=1e-12)


def test_rope_partial_rotary_dim_leaves_tail():
    x = np.arange(1.0, 9.0)
    y = rope_rotate(x, 5, 1e4, rotary_dim=4)
    np.testing.assert_array_equal(y[4:], x[4:])
    np.testing.assert_allclose(y[:4], rope_rotate(x[:4], 5, 1e4), atol=1e-15)


def test_rope_identity_norm_composition_relative():
    r = np.random.default_rng(30)
    x = r.standard_normal((6, 128))
    np.testing.assert_array_equal(rope_rotate(x, 0, 1e6), x)
    for a, b in [(3, 5), (1000, 65000), (123456, 7)]:
        ya = rope_rotate(x, a, 1e6)
        np.testing.assert_allclose(np.linalg.norm(ya, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
        np.testing.assert_allclose(rope_rotate(ya, b, 1e6), rope_rotate(x, a + b, 1e6), atol=1e-10)
        q, k = x[0], x[1]
        d1 = rope_rotate(q, a, 1e6) @ rope_rotate(k, b, 1e6)
        d2 = rope_rotate(q, a + 17, 1e6) @ rope_rotate(k, b + 17, 1e6)
        assert abs(d1 - d2) < 1e-9


def _delta_bar(o):
    """Bound on |R(dp) bf16(R(p_old) x) - bf16(R(p_new) x)| per element, both
    sides rounded to bf16 at the end.

    The baked K carries one rounding error per element, at most half a bf16
    ULP, i.e. 2^-8 of the element; as a vector over the rotation pair that is
    at most 2^-8 (1 + 2^-8) of the pair's magnitude, and the rotation by dp
    moves it, unchanged in length, onto both components.  The two final
    roundings of values that close differ by at most one step of the
    element's own grid (its ULP) plus that carried error, which the ULP grid
    of the larger of the two values stretches by at most 2^-7 of itself."""
    return bf16_ulp(o) + 2.0 ** -8 * (1 + 2.0 ** -8) * (1 + 2.0 ** -7) * pair_norm(o)


# ---------------------------------------------------------------- gather

def test_gather_plain_copies_bit_for_bit():
    r = np.random.default_rng(31)
    bt, D, NB = 3, 4, 7
    sk = numerics.round_to_bf16(r.standard_normal((NB * bt, D)))
    sv = numerics.round_to_bf16(r.standard_normal((NB * bt, D)))
    idx = np.array([0, 2, 3, 6])
    k, v = om.gather_view(sk, sv, idx, bt)
    for i, b in enumerate(idx):
        for o in range(bt):
            assert np.array_equal(k[i * bt + o], sk[b * bt + o])
            assert np.array_equal(v[i * bt + o], sv[b * bt + o])


def test_gather_raw_rerope_equals_baked_at_new_position():
    # raw K re-rotated at its new slot equals K baked at that position
    r = np.random.default_rng(32)
    bt, D, NB = 4, 8, 6
    raw = numerics.round_to_bf16(r.standard_normal((NB * bt, D)))
    idx = np.array([1, 4, 5])
    k, v = om.gather_view(raw, raw, idx, bt, rope="raw", theta=1e6, pos0=10)
    for i, b in enumerate(idx):
        for o in range(bt):
            baked = rope_rotate(raw[b * bt + o], 10 + i * bt + o, 1e6)
            np.testing.assert_array_equal(k[i * bt + o], numerics.round_to_bf16(baked))
    np.testing.assert_array_equal(v, raw[(idx[:, None] * bt + np.arange(bt)).ravel()])


def test_gather_delta_on_baked_matches_raw_within_two_ulp():
    r = np.random.default_rng(33)
    bt, D, NB = 32, 128, 40
    raw = numerics.round_to_bf16(r.standard_normal((NB * bt, D)))
    baked = numerics.round_to_bf16(rope_rotate(raw, np.arange(NB * bt), 1e6))
    idx = np.array([0, 3, 17, 39])
    k_raw, _ = om.gather_view(raw, raw, idx, bt, rope="raw")
    k_del, _ = om.gather_view(baked, baked, idx, bt, rope="delta")
    assert np.all(np.abs(k_del - k_raw) <= _delta_bar(k_raw))


# ---------------------------------------------------------------- incremental view

def _incremental_case(seed, nb=60, k=12, overlap=6, bt=4, D=8, spare=3):
    r = np.random.default_rng(seed)
    raw_k = numerics.round_to_bf16(r.standard_normal((nb, bt, D)))
    raw_v = numerics.round_to_bf16(r.standard_normal((nb, bt, D)))
    new_idx = np.sort(r.choice(nb, k, replace=False))
    outside = np.setdiff1d(np.arange(nb), new_idx)
    prev_idx = np.sort(np.concatenate([r.choice(new_idx, overlap, replace=False),
                                       r.choice(outside, k - overlap, replace=False)]))
    P = k + spare
    prev_page = r.permutation(P)[:k]
    pool_k = numerics.round_to_bf16(r.standard_normal((P, bt, D)))
    pool_v = numerics.round_to_bf16(r.standard_normal((P, bt, D)))
    o = np.arange(bt)
    for i, b in enumerate(prev_idx):               # previous view: baked at its old slots
        pool_k[prev_page[i]] = numerics.round_to_bf16(rope_rotate(raw_k[b], i * bt + o, 1e6))
        pool_v[prev_page[i]] = raw_v[b]
    return raw_k, raw_v, new_idx, prev_idx, prev_page, pool_k, pool_v


@pytest.mark.parametrize("seed", [40, 41, 42])
def test_incremental_equals_fresh_build(seed):
    raw_k, raw_v, new_idx, prev_idx, prev_page, pool_k, pool_v = _incremental_case(seed)
    bt, D = raw_k.shape[1], raw_k.shape[2]
    pk, pv, pt, n_miss = om.incremental_view(prev_idx, prev_page, new_idx, pool_k, pool_v,
                                             raw_k, raw_v, bt, theta=1e6)
    fk, fv = om.gather_view(raw_k.reshape(-1, D), raw_v.reshape(-1, D), new_idx, bt, rope="raw")
    view_k = pk[pt].reshape(-1, D)
    view_v = pv[pt].reshape(-1, D)
    np.testing.assert_array_equal(view_v, fv)
    assert np.all(np.abs(view_k - fk) <= _delta_bar(fk))
    hits = np.intersect1d(prev_idx, new_idx)
    assert n_miss == len(new_idx) - len(hits)
    assert len(set(pt.tolist())) == len(pt)                       # each page once
    freed = set(prev_page[~np.isin(prev_idx, new_idx)].tolist())
    hit_pages = set(prev_page[np.isin(prev_idx, new_idx)].tolist())
    miss_pages = set(pt[~np.isin(new_idx, prev_idx)].tolist())
    assert not (hit_pages & freed) and miss_pages == freed        # misses fill freed pages
    # untouched pages keep their bytes
    other = np.setdiff1d(np.arange(pool_k.shape[0]), pt)
    np.testing.assert_array_equal(pk[other], pool_k[other])


@pytest.mark.parametrize("seed", [44, 45])
def test_incremental_raw_hits_equal_a_fresh_build_bit_for_bit(seed):
    # moved hits re-rotated from raw K: the whole view is the fresh raw gather
    raw_k, raw_v, new_idx, prev_idx, prev_page, pool_k, pool_v = _incremental_case(seed)
    bt, D = raw_k.shape[1], raw_k.shape[2]
    pk, pv, pt, n_miss = om.incremental_view(prev_idx, prev_page, new_idx, pool_k, pool_v,
                                             raw_k, raw_v, bt, theta=1e6, hits="raw")
    fk, fv = om.gather_view(raw_k.reshape(-1, D), raw_v.reshape(-1, D), new_idx, bt, rope="raw")
    np.testing.assert_array_equal(pk[pt].reshape(-1, D), fk)
    np.testing.assert_array_equal(pv[pt].reshape(-1, D), fv)
    pk_d, _, pt_d, n_d = om.incremental_view(prev_idx, prev_page, new_idx, pool_k, pool_v,
                                             raw_k, raw_v, bt, theta=1e6)
    np.testing.assert_array_equal(pt_d, pt)
    assert n_d == n_miss
    with pytest.raises(ValueError):
        om.incremental_view(prev_idx, prev_page, new_idx, pool_k, pool_v, raw_k, raw_v, bt, hits="both")


def test_incremental_delta_hits_drift_over_steps_raw_hits_do_not():
    """The drift of in-place delta rotation, step after step, against raw K
    rotated once at the block's current position (D 128, 32-token blocks,
    theta 1e6, a block that moves at every step).  One delta step carries
    one extra bf16 rounding (relative row error about 2^-9 per rounding);
    the errors of successive steps add up, while re-rotating from raw K
    keeps every step at one rounding of the exact rotation."""
    r = np.random.default_rng(46)
    bt, D, nb, k = 32, 128, 64, 16
    raw_k = numerics.round_to_bf16(r.standard_normal((nb, bt, D)))
    raw_v = numerics.round_to_bf16(r.standard_normal((nb, bt, D)))
    o = np.arange(bt)
    target = 40                                    # stays selected; other blocks come and go before it
    sel = np.sort(np.concatenate([[target], r.choice(np.setdiff1d(np.arange(nb), [target]), k - 1, replace=False)]))
    page = np.arange(k)
    state = {}
    for hits in ("delta", "raw"):
        pool_k = np.zeros((k, bt, D))
        pool_v = np.zeros((k, bt, D))
        for i, b in enumerate(sel):
            pool_k[i] = numerics.round_to_bf16(rope_rotate(raw_k[b], i * bt + o, 1e6))
            pool_v[i] = raw_v[b]
        prev, prev_page, errs = sel, page, []
        rs = np.random.default_rng(47)
        for step in range(8):
            below = np.arange(target)
            lo = rs.choice(below, rs.integers(3, 12), replace=False)     # how many blocks precede the target
            hi = np.setdiff1d(np.arange(target + 1, nb), [])
            rest = rs.choice(hi, k - 1 - len(lo), replace=False)
            new = np.sort(np.concatenate([lo, [target], rest]))
            pool_k, pool_v, pt, _ = om.incremental_view(prev, prev_page, new, pool_k, pool_v, raw_k, raw_v, bt,
                                                        theta=1e6, hits=hits)
            i_t = int(np.searchsorted(new, target))
            exact = rope_rotate(raw_k[target], i_t * bt + o, 1e6)
            got = pool_k[pt[i_t]]
            errs.append(float(np.linalg.norm(got - exact) / np.linalg.norm(exact)))
            prev, prev_page = new, pt
        state[hits] = errs
    one = 2.0 ** -9 * np.sqrt(1.0)                 # a single bf16 rounding's relative row error is about this
    assert max(state["raw"]) < 1.6 * one           # every step: one rounding of the exact rotation
    assert state["delta"][-1] > 1.5 * max(state["raw"])   # eight moves: several roundings accumulated
    assert state["delta"][-1] > state["delta"][0]


def test_incremental_unmoved_hit_is_bitwise():
    raw_k, raw_v, new_idx, prev_idx, prev_page, pool_k, pool_v = _incremental_case(43, overlap=12)
    pk, pv, pt, n_miss = om.incremental_view(prev_idx, prev_page, new_idx, pool_k, pool_v,
                                             raw_k, raw_v, raw_k.shape[1])
    assert n_miss == 0
    np.testing.assert_array_equal(pk, pool_k)
    np.testing.assert_array_equal(pv, pool_v)


# ---------------------------------------------------------------- redirect and dead slot

def test_redirect_invariants():
    r = np.random.default_rng(50)
    N, dead = 64, 999
    sm = r.permutation(N * 2)[:N]
    sm[[3, 9]] = dead
    keep = r.random(N) > 0.5
    keep[[3]] = True                                   # a kept-but-dead entry stays dead
    out = om.redirect(sm, keep, dead)
    np.testing.assert_array_equal(out[keep], sm[keep])
    assert np.all(out[~keep] == dead)
    assert out[3] == dead and out[9] == dead
    np.testing.assert_array_equal(om.redirect(out, keep, dead), out)     # idempotent


def _dead_slot_case(q_sign, D=128, N=40, seed=51):
    r = np.random.default_rng(seed)
    kb, vb = om.sentinel_rows("bf16", D)
    n_slots = N + 1
    dead = N
    pool_k = numerics.round_to_bf16(r.standard_normal((n_slots, D)))
    pool_v = numerics.round_to_bf16(r.standard_normal((n_slots, D)))
    pool_k[dead], pool_v[dead] = kb, vb
    slot_map = np.arange(N)
    keep = r.random(N) > 0.4
    redirected = om.redirect(slot_map, keep, dead)
    q = r.standard_normal(D) * 0.1 + q_sign * 0.05
    return q, pool_k, pool_v, slot_map, redirected, keep, dead


def test_decode_attention_two_key_closed_form():
    # D = 4, q = (2,0,0,0): logits q.k/sqrt(4) are 1 for k0 = e0 and 0 for k1 = 0,
    # so o = (e v0 + v1) / (e + 1); the slot map reads slots 3 and 1
    pool_k = np.zeros((4, 4)); pool_k[3, 0] = 1.0
    pool_v = np.zeros((4, 4)); pool_v[3] = [1.0, 2.0, 0.0, 0.0]; pool_v[1] = [0.0, 0.0, 4.0, 8.0]
    q = np.array([2.0, 0.0, 0.0, 0.0])
    e = math.e
    want = (e * pool_v[3] + pool_v[1]) / (e + 1)
    np.testing.assert_allclose(om.decode_attention_slots(q, pool_k, pool_v, [3, 1]), want, atol=1e-15)
    np.testing.assert_allclose(om.decode_attention_hard(q, pool_k, pool_v, [3, 1, 2], [1, 1, 0]), want,
                               atol=1e-15)


@pytest.mark.parametrize("q_sign", [1.0, -1.0, 0.0])
def test_dead_slot_closed_form(q_sign):
    q, pool_k, pool_v, slot_map, redirected, keep, dead = _dead_slot_case(q_sign)
    D = q.shape[0]
    o_dead = om.decode_attention_slots(q, pool_k, pool_v, redirected)
    o_hard = om.decode_attention_hard(q, pool_k, pool_v, slot_map, keep)
    logits = pool_k[slot_map[keep]] @ q / math.sqrt(D)
    l_dead = -9984.0 * q.sum() / math.sqrt(D)
    m = max(logits.max(), l_dead)
    z = np.exp(logits - m).sum()
    n_dead = int((~keep).sum())
    factor = z / (z + n_dead * math.exp(l_dead - m))
    np.testing.assert_allclose(o_dead, o_hard * factor, rtol=1e-12, atol=1e-15)


def test_dead_slot_is_a_hard_mask_only_with_margin():
    # sum(q) large and positive: the sentinel's weight underflows -> equal bitwise
    q, pool_k, pool_v, slot_map, redirected, keep, dead = _dead_slot_case(1.0)
    q = q + 0.5
    o_dead = om.decode_attention_slots(q, pool_k, pool_v, redirected)
    o_hard = om.decode_attention_hard(q, pool_k, pool_v, slot_map, keep)
    np.testing.assert_array_equal(o_dead, o_hard)
    # sum(q) < 0: the sentinel logit is large and positive; V = 0 rows swamp
    # the softmax, so the output collapses toward zero rather than matching
    q2 = -np.abs(q)
    o2 = om.decode_attention_slots(q2, pool_k, pool_v, redirected)
    h2 = om.decode_attention_hard(q2, pool_k, pool_v, slot_map, keep)
    assert np.linalg.norm(o2) < 1e-6 * np.linalg.norm(h2)


# ---------------------------------------------------------------- alias-aware free list

def test_free_list_hand_example():
    # slots: j0 5 (kept), j1 6 (dropped, but j2 keeps 6: aliased), j3 7 (freed),
    # j4 dead (prior redirect), j5 9 (freed), j6 5 (dropped, kept by j0), j7 10 (kept),
    # j8 and j9 both 11 (dropped twice: freed once)
    D = 99
    sm = [5, 6, 6, 7, D, 9, 5, 10, 11, 11]
    keep = [1, 0, 1, 0, 0, 0, 0, 1, 0, 0]
    np.testing.assert_array_equal(om.free_list(sm, keep, D), [7, 9, 11])
    # a radix-protected prefix of 4 positions keeps slot 7 (position 3) allocated;
    # a prefix of 3 stops just before it
    np.testing.assert_array_equal(om.free_list(sm, keep, D, protected_len=4), [9, 11])
    np.testing.assert_array_equal(om.free_list(sm, keep, D, protected_len=3), [7, 9, 11])
    # nothing dropped, or everything protected: nothing freed
    assert om.free_list(sm, [1] * 10, D).size == 0
    assert om.free_list(sm, keep, D, protected_len=10).size == 0


def test_reusing_freed_slots_never_changes_a_kept_or_sibling_read():
    # Two requests share a radix-protected prefix of physical slots; each has
    # its own tail, with aliases from earlier rounds.  After request 0 drops
    # entries and its freed slots are handed to new data, every position that
    # request 0 keeps and every position of request 1 reads what it read before.
    rng = np.random.default_rng(3)
    dead = 1000
    pool = rng.standard_normal((dead + 1, 4))
    P = 16
    prefix = rng.permutation(200)[:P]
    tail0 = rng.integers(200, 400, size=48)          # duplicates: slots shared inside the tail
    tail1 = rng.integers(400, 600, size=48)
    sm0 = np.concatenate([prefix, tail0]); sm1 = np.concatenate([prefix, tail1])
    sm0[rng.choice(np.arange(P, 64), 6, replace=False)] = dead   # redirected in an earlier round
    keep0 = rng.random(64) < 0.4
    keep0[sm0 == dead] = False
    before0 = pool[sm0[keep0]].copy(); before1 = pool[sm1].copy()
    freed = om.free_list(sm0, keep0, dead, protected_len=P)
    assert dead not in freed and not set(freed) & set(prefix.tolist())
    pool2 = pool.copy()
    pool2[freed] = 12345.0                            # the allocator hands them out again
    np.testing.assert_array_equal(pool2[sm0[keep0]], before0)
    np.testing.assert_array_equal(pool2[sm1], before1)
    # and every slot that only dropped, unprotected positions referenced is freed
    only_dropped = set(sm0[P:][~keep0[P:]].tolist()) - set(sm0[keep0].tolist()) - {dead}
    assert set(freed.tolist()) == only_dropped


# ---------------------------------------------------------------- tail compaction

def test_tail_compact_hand_example():
    # bs = 4, Y = 4 blocks (physical 7, 2, 9, 5), N = 14 positions, 6 kept:
    # X = ceil(6/4) = 2, target = logical blocks 2..3 = slots 8..15.
    # kept 0, 3, 6 (sources), 9, 10, 13 (stay); destinations: 8, 11, 12
    # (14, 15 are empty slots past N and remain unused).
    keep = np.zeros(14, bool); keep[[0, 3, 6, 9, 10, 13]] = True
    bt = [7, 2, 9, 5]
    pool_k = np.arange(10 * 4, dtype=np.float64).reshape(10, 4, 1)
    pool_v = -pool_k
    kp, vp, slot_pos, freed = om.tail_compact(keep, bt, 4, pool_k, pool_v)
    np.testing.assert_array_equal(freed, [7, 2])
    want_pos = [-1] * 8 + [0, 9, 10, 3, 6, 13, -1, -1]
    np.testing.assert_array_equal(slot_pos, want_pos)
    # slot 8 = physical (9, 0) now holds position 0 = physical (7, 0); slot 11 =
    # (9, 3) holds position 3 = (7, 3); slot 12 = (5, 0) holds position 6 = (2, 2)
    assert kp[9, 0, 0] == pool_k[7, 0, 0] and kp[9, 3, 0] == pool_k[7, 3, 0]
    assert kp[5, 0, 0] == pool_k[2, 2, 0] and vp[5, 0, 0] == pool_v[2, 2, 0]
    # everything else is untouched
    changed = np.argwhere(kp[..., 0] != pool_k[..., 0])
    assert sorted(map(tuple, changed)) == [(5, 0), (9, 0), (9, 3)]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tail_compact_preserves_kept_entries(seed):
    rng = np.random.default_rng(seed)
    bs, Y = 16, 24
    N = Y * bs - rng.integers(0, bs)
    keep = rng.random(N) < rng.uniform(0.2, 0.9)
    keep[-16:] = True                                   # recent entries forced, as a selection would
    P = 64
    bt = rng.permutation(P)[:Y]
    pool_k = rng.standard_normal((P, bs, 3)); pool_v = rng.standard_normal((P, bs, 3))
    kp, vp, slot_pos, freed = om.tail_compact(keep, bt, bs, pool_k, pool_v)
    n_kept = int(keep.sum()); X = -(-n_kept // bs)
    assert len(freed) == Y - X and set(freed) == set(bt[: Y - X])
    # the multiset of kept (position, K, V) equals what the target region holds
    held = slot_pos[slot_pos >= 0]
    assert sorted(held.tolist()) == np.flatnonzero(keep).tolist()
    assert np.all(slot_pos[: (Y - X) * bs] == -1)
    for s in np.flatnonzero(slot_pos >= 0):
        p = slot_pos[s]
        np.testing.assert_array_equal(kp[bt[s // bs], s % bs], pool_k[bt[p // bs], p % bs])
        np.testing.assert_array_equal(vp[bt[s // bs], s % bs], pool_v[bt[p // bs], p % bs])
    # blocks outside the request are untouched
    others = np.setdiff1d(np.arange(P), bt)
    np.testing.assert_array_equal(kp[others], pool_k[others])
