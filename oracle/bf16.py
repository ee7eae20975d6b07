"""bfloat16 rounding written out from the format's definition (oracle).

bfloat16 = 1 sign bit, 8 exponent bits (same range as IEEE binary32),
7 stored fraction bits, i.e. 8 significant bits for normal numbers.
Round-to-nearest, ties-to-even ("RNE") is the rounding the method's bf16 K/V
storage uses.  The rounding is done directly from float64 (no intermediate
binary32 step, so there is no double rounding).
"""
from __future__ import annotations

import numpy as np

# Largest finite bfloat16: (2 - 2**-7) * 2**127.
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
# Quantum of the bfloat16 subnormal range (same minimum exponent as binary32).
_SUBNORMAL_QUANTUM_EXP = -133


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even).

    Returns float64 values that are exactly representable in bfloat16.
    A value with leading bit 2**(e-1) has quantum 2**(e-8) (8 significant
    bits); below the normal range the quantum is fixed at 2**-133.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    q_exp = np.maximum(e.astype(np.int64) - 8, _SUBNORMAL_QUANTUM_EXP)
    q = np.ldexp(1.0, q_exp)
    r = np.rint(x / q) * q                  # np.rint: round half to even
    r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, x), r)
    return np.where(np.isnan(x), x, r)


def bf16_ulp(x) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (the unit in the last place)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(x)
    q_exp = np.maximum(e.astype(np.int64) - 8, _SUBNORMAL_QUANTUM_EXP)
    return np.ldexp(1.0, q_exp)


def bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bits(x) -> np.ndarray:
    """float64 values that are exact bfloat16 -> uint16 bit patterns."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    if not np.array_equal(f.astype(np.float64), x, equal_nan=True):
        raise ValueError("values are not representable in bfloat16")
    u = f.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("values are not representable in bfloat16")
    return (u >> np.uint32(16)).astype(np.uint16)


def ulp_distance(a, b) -> np.ndarray:
    """Number of bfloat16 steps between two arrays of bfloat16 values.

    Maps each bit pattern to a signed integer that is monotone in the value
    (magnitude bits, negated for negative numbers; +0 and -0 both map to 0).
    """
    def ordered(v):
        u = f64_to_bits(v).astype(np.int32)
        mag = u & 0x7FFF
        return np.where(u & 0x8000, -mag, mag)

    return np.abs(ordered(a) - ordered(b))
