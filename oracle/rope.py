"""Rotary position embedding, float64.  Test infrastructure only.

KVMem (tiered movement): K with RoPE baked in is invalid once a block moves
to a new logical position, so a position-independent raw K is rotated at the
new position when the view is built.  The pages do not fix the RoPE
convention; the reading taken here is the rotate-half form with
inv_freq[m] = theta ** (-2m / rotary_dim), pairs (m, m + rotary_dim/2), and
dimensions past ``rotary_dim`` left as they are.  ``style="interleaved"``
pairs (2m, 2m+1) instead.  Angles are p * inv_freq with integer p, in float64.
"""
import numpy as np


def inv_freq(rotary_dim, theta):
    m = np.arange(rotary_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * m / rotary_dim)


def rope_rotate(x, pos, theta, style="half", rotary_dim=None):
    """Rotate the last axis of ``x`` by position ``pos`` (broadcast over rows).

    For pair (a, b) with angle phi = pos * inv_freq[m]:
    (a, b) -> (a cos phi - b sin phi, a sin phi + b cos phi).
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    rd = D if rotary_dim is None else rotary_dim
    half = rd // 2
    f = inv_freq(rd, theta)
    p = np.asarray(pos, dtype=np.float64)[..., None]            # exact for |p| < 2**53
    phi = p * f
    c, s = np.cos(phi), np.sin(phi)
    out = x.copy()
    if style == "half":
        a, b = x[..., :half], x[..., half:rd]
        out[..., :half] = a * c - b * s
        out[..., half:rd] = a * s + b * c
    elif style == "interleaved":
        a, b = x[..., 0:rd:2], x[..., 1:rd:2]
        out[..., 0:rd:2] = a * c - b * s
        out[..., 1:rd:2] = a * s + b * c
    else:
        raise ValueError(style)
    return out
