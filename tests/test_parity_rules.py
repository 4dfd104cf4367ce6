"""The acceptance rules of tests/parity.py, checked on the CPU.

The re-RoPE bar must tell an accurately reduced rotation from the hazard it
exists to catch: rotating at large positions with the angle formed in
float32 (the product p * inv_freq rounded to 24 bits loses up to p * 2^-24
radians).  KVMem (tiered movement) re-RoPEs raw keys at their new contiguous
view positions, which reach 131072 in the 10M-token view; every emulation
below rotates bf16 rows at positions spread over [0, 131072) with theta 1e6
and D 128, and compares the bf16 result with the oracle's float64 rotation
rounded once.
"""
import numpy as np
import pytest

from oracle import numerics
from oracle.rope import inv_freq, rope_rotate
from parity import (Conditioning, assert_rope_close, bf16_ulp, block_score_tolerance, boundary_gap, gamma32,
                    pair_norm, qbar_error_bound, rope_violations)

D, THETA = 128, 1e6


def _rows(seed, n):
    r = np.random.default_rng(seed)
    x = numerics.round_to_bf16(r.standard_normal((n, D)))
    p = np.concatenate([r.integers(0, 131072, n - 64), np.arange(131072 - 64, 131072)])
    return x, p


def _rotate_f32(x, cos32, sin32):
    """Rotate-half in float32 arithmetic given float32 cos/sin per pair, one
    fused multiply-add per output element, rounded once to bf16."""
    h = D // 2
    a = x[:, :h].astype(np.float32)
    b = x[:, h:].astype(np.float32)
    ac = (a * cos32).astype(np.float64)
    bc = (b * cos32).astype(np.float64)
    first = (ac - b.astype(np.float64) * sin32.astype(np.float64)).astype(np.float32)
    second = (bc + a.astype(np.float64) * sin32.astype(np.float64)).astype(np.float32)
    return numerics.round_to_bf16(np.concatenate([first, second], axis=1).astype(np.float64))


def _reduced_angle_rotation(x, p):
    """The angle p * inv_freq formed in float64 and reduced modulo 2 pi in
    float64, then float32 cos/sin and float32 products."""
    phi = p[:, None].astype(np.float64) * inv_freq(D, THETA)[None]
    r = phi - np.rint(phi / (2 * np.pi)) * (2 * np.pi)
    r32 = r.astype(np.float32)
    return _rotate_f32(x, np.cos(r32), np.sin(r32))


def _fp32_angle_rotation(x, p):
    """The hazard: the angle formed as a float32 product."""
    phi32 = p[:, None].astype(np.float32) * inv_freq(D, THETA)[None].astype(np.float32)
    return _rotate_f32(x, np.cos(phi32), np.sin(phi32))


def _oracle(x, p):
    return numerics.round_to_bf16(rope_rotate(x, p, THETA))


def test_rope_bar_accepts_accurately_reduced_float32_rotation():
    x, p = _rows(1, 4096)
    assert_rope_close(_reduced_angle_rotation(x, p), _oracle(x, p))


def test_rope_bar_rejects_float32_angles():
    x, p = _rows(2, 4096)
    bad = rope_violations(_fp32_angle_rotation(x, p), _oracle(x, p))
    assert bad.sum() > 1000
    with pytest.raises(AssertionError):
        assert_rope_close(_fp32_angle_rotation(x, p), _oracle(x, p))


def test_rope_bar_rejects_a_position_off_by_one():
    x, p = _rows(3, 512)
    with pytest.raises(AssertionError):
        assert_rope_close(_reduced_angle_rotation(x, p + 1), _oracle(x, p))


def test_rope_bar_rejects_one_ulp_too_many_on_one_element():
    x, p = _rows(4, 64)
    o = _oracle(x, p)
    g = o.copy()
    i = np.argmax(np.abs(o) / np.maximum(pair_norm(o), 1e-30))   # an element that dominates its pair
    g.flat[i] += 2 * bf16_ulp(o.flat[i])
    with pytest.raises(AssertionError):
        assert_rope_close(g, o)


def test_pair_norm_follows_the_pairing():
    x = np.arange(8, dtype=np.float64)[None]
    np.testing.assert_allclose(pair_norm(x, "half")[0, :4], np.hypot(x[0, :4], x[0, 4:]))
    np.testing.assert_allclose(pair_norm(x, "interleaved")[0, ::2], np.hypot(x[0, ::2], x[0, 1::2]))


def test_bf16_ulp_grid():
    assert bf16_ulp(1.0) == 2.0 ** -7 and bf16_ulp(1.99) == 2.0 ** -7 and bf16_ulp(2.0) == 2.0 ** -6
    assert bf16_ulp(-0.75) == 2.0 ** -8 and bf16_ulp(0.0) == 0.0


# ---------------------------------------------------------------- block-score bound

def test_gamma32_bounds_float32_summation_in_any_order():
    r = np.random.default_rng(5)
    for n in (2, 17, 256, 4096):
        t = (r.standard_normal(n) * np.exp(r.standard_normal(n) * 3)).astype(np.float32)
        exact = float(np.sum(t.astype(np.float64)))
        for order in (np.arange(n), r.permutation(n)):
            acc = np.float32(0.0)
            for v in t[order]:
                acc = np.float32(acc + v)
            assert abs(float(acc) - exact) <= gamma32(n) * float(np.abs(t.astype(np.float64)).sum())


def test_block_score_tolerance_covers_a_float32_hi_lo_dot_and_rejects_a_dropped_term():
    # q-bar as float32 split into f16 hi + lo parts after a power-of-two scaling,
    # products with the f16 index summed in float32: the block scorer's arithmetic
    r = np.random.default_rng(6)
    Dd, n = 128, 400
    qbar = (r.standard_normal(Dd) * 300).astype(np.float32)
    mu = (r.standard_normal((n, Dd)) * 0.2).astype(np.float16)
    scale = 1 / np.sqrt(Dd)
    e2 = np.frexp(np.abs(qbar).max())[1]
    x = qbar * np.float32(2.0 ** (14 - e2))
    hi = x.astype(np.float16)
    lo = (x - hi.astype(np.float32)).astype(np.float16)
    got = np.empty(n)
    for b in range(n):
        acc = np.float32(0)
        for d in range(Dd):
            acc = np.float32(acc + np.float32(hi[d]) * np.float32(mu[b, d]))
            acc = np.float32(acc + np.float32(lo[d]) * np.float32(mu[b, d]))
        got[b] = float(np.float32(acc * np.float32(scale * 2.0 ** (e2 - 14))))
    q64, mu64 = qbar.astype(np.float64), mu.astype(np.float64)
    want = mu64 @ q64 * scale
    tol = block_score_tolerance(want, np.abs(q64), mu64, scale, qbar_err=np.zeros(Dd))
    assert np.all(np.abs(got - want) <= tol)
    dropped = want - mu64[:, 5] * q64[5] * scale
    assert np.any(np.abs(dropped - want) > tol)


def test_qbar_error_bound_covers_float64_summation_rounded_once():
    r = np.random.default_rng(7)
    q = numerics.round_to_bf16(r.standard_normal((4096, 16)) + 0.2)
    exact = q.sum(axis=0)
    got = np.float32(np.cumsum(q, axis=0)[-1]).astype(np.float64)     # float64 sum, one rounding
    bound = qbar_error_bound(np.abs(exact), np.abs(q).sum(axis=0), 4096)
    assert np.all(np.abs(got - exact) <= bound)
    # a float32 running sum is not held to it
    acc = np.zeros(16, np.float32)
    for row in q.astype(np.float32):
        acc = (acc + row).astype(np.float32)
    assert np.any(np.abs(acc.astype(np.float64) - exact) > bound)


def test_boundary_gap_and_conditioning_counts():
    s = np.array([9.0, 1.0, 5.0, 5.0, 3.0, 2.0, 8.0, 7.0])      # forced: 0 (sink) and 7 (recent)
    assert boundary_gap(s, 4, 1, 1) == 0.0                      # 2 of {1..6} by score: 5 and 5 tie at the edge
    assert boundary_gap(s, 5, 1, 1) == (5.0 - 3.0) / 5.0        # 3 of them: 8, 5, 5 kept, 3 out
    assert boundary_gap(s, 8, 1, 1) is None                     # everything fits
    alive = np.array([1, 1, 0, 1, 1, 1, 1, 1], bool)
    assert boundary_gap(s, 4, 1, 1, alive) == (5.0 - 3.0) / 5.0
    c = Conditioning("x")
    c.add("exact", 0.5)
    c.add("near-tie", 0.0)
    c.add("exact", 1e-7)
    c.add("exact", None)
    assert (c.units, c.exact, c.accepted, c.near, c.ties) == (4, 3, 1, 2, 1)
    assert "4 units compared" in c.report()
