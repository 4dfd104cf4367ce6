"""Rounding of float64 results to the storage formats the GPU path writes.

Test infrastructure only (see ``oracle/__init__``).

Each routine rounds a float64 value ONCE, round-to-nearest-even, to the target
format, so the oracle never double-rounds through an intermediate format.
bfloat16 keeps 8 significant bits and float32's exponent range; float16 keeps
11 significant bits with exponents down to 2**-14 (subnormals to 2**-24).
"""
import numpy as np


def _round_sig(x, sig_bits, min_quantum_exp, overflow_at):
    """Round float64 ``x`` to ``sig_bits`` significant bits (RNE).

    ``min_quantum_exp``: exponent of the spacing of the subnormal range.
    ``overflow_at``: smallest magnitude that is no longer finite after rounding.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e = np.frexp(xf)                      # xf = m * 2**e, 0.5 <= |m| < 1
    q_exp = np.maximum(e - sig_bits, min_quantum_exp)
    q = np.ldexp(1.0, q_exp)
    r = np.rint(xf / q) * q                  # division by a power of two is exact
    r = np.where(np.abs(r) >= overflow_at, np.copysign(np.inf, r), r)
    out[fin] = r
    return out


def round_to_bf16(x):
    """float64 -> nearest bfloat16 value (returned as float64)."""
    return _round_sig(x, 8, -133, 2.0 ** 128)


def round_to_f16(x):
    """float64 -> nearest IEEE half value (returned as float64)."""
    return _round_sig(x, 11, -24, 65520.0)


def round_to_f32(x):
    """float64 -> nearest float32 (NumPy's cast is a single RNE rounding)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_bits(x):
    """Bit pattern (uint16) of values already representable in bfloat16."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def f16_bits(x):
    """Bit pattern (uint16) of values already representable in float16."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def bf16_from_bits(bits):
    """uint16 bfloat16 bit patterns -> float64 values."""
    b = np.asarray(bits, dtype=np.uint32) << 16
    return b.astype(np.uint32).view(np.float32).astype(np.float64)
