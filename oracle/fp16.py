"""IEEE binary16 ("fp16") rounding written out from the format's definition
(oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The voxtral.c explainer's file table (section 七) points to an fp16 KV cache
(SPEED.md); the cache variant that stores K and V as fp16 rounds every stored
value this way.  binary16 = 1 sign bit, 5 exponent bits (bias 15), 10 stored
fraction bits: 11 significant bits for normal numbers, largest finite value
65504, subnormal quantum 2**-24.  Round to nearest, ties to even, directly
from float64 (no binary32 step, so no double rounding); values at or beyond
65520 in magnitude overflow to infinity, as IEEE round-to-nearest requires.
"""
from __future__ import annotations

import numpy as np

F16_MAX = 65504.0
_SUBNORMAL_QUANTUM_EXP = -24
_SIGNIFICANT_BITS = 11


def round_f16(x) -> np.ndarray:
    """Round float64 values to the nearest binary16 value (ties to even).

    A value with leading bit 2**(e-1) has quantum 2**(e-11); below the normal
    range (2**-14) the quantum stays 2**-24.  Returns float64 values exactly
    representable in binary16.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    q_exp = np.maximum(e.astype(np.int64) - _SIGNIFICANT_BITS, _SUBNORMAL_QUANTUM_EXP)
    q = np.ldexp(1.0, q_exp)
    r = np.rint(x / q) * q                  # np.rint: round half to even
    r = np.where(np.abs(r) > F16_MAX, np.copysign(np.inf, x), r)
    return np.where(np.isnan(x), x, r)


def f16_ulp(x) -> np.ndarray:
    """Spacing of binary16 numbers at |x|."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(x)
    q_exp = np.maximum(e.astype(np.int64) - _SIGNIFICANT_BITS, _SUBNORMAL_QUANTUM_EXP)
    return np.ldexp(1.0, q_exp)


def bits_to_f64(bits) -> np.ndarray:
    """binary16 bit patterns (uint16) -> float64 values (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f64_to_bits(x) -> np.ndarray:
    """float64 values that are exact binary16 -> uint16 bit patterns."""
    x = np.asarray(x, dtype=np.float64)
    h = x.astype(np.float16)
    if not np.array_equal(h.astype(np.float64), x, equal_nan=True):
        raise ValueError("values are not representable in binary16")
    return h.view(np.uint16)


def ulp_distance(a, b) -> np.ndarray:
    """Number of binary16 steps between two arrays of binary16 values."""
    def ordered(v):
        u = f64_to_bits(v).astype(np.int32)
        mag = u & 0x7FFF
        return np.where(u & 0x8000, -mag, mag)

    return np.abs(ordered(a) - ordered(b))
