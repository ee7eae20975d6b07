"""Rotary position embedding and its exact rotation matrices (oracle).

The Audio8 explainer ("Rolling KV Cache 三步拆解", step 2) says every K carries
its absolute position through RoPE, and that re-basing subtracts the evicted
offset from all retained K with the exact rotation matrix rather than an
approximate correction.  The pages do not fix the pairing convention, the
frequency schedule or the base; this oracle takes the standard RoPE
frequencies theta_i = base**(-2i/d), i in [0, d/2), and pairs element i with
element i + d/2 ("half-split"), with base 1e6 for the decoder workloads.

R(p) rotates each pair (x_i, x_{i+d/2}) by the angle p * theta_i:

    y_i       = x_i cos(p theta_i) - x_{i+d/2} sin(p theta_i)
    y_{i+d/2} = x_i sin(p theta_i) + x_{i+d/2} cos(p theta_i)

so R(a) R(b) = R(a + b) and R(-D) applied to R(p) x gives R(p - D) x, the
identity that makes re-basing exact in real arithmetic.
"""
from __future__ import annotations

import numpy as np


def inv_freq(d: int, base: float) -> np.ndarray:
    """theta_i = base ** (-2 i / d) for i in [0, d/2), float64."""
    if d % 2:
        raise ValueError("head dim must be even")
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / d)


def angles(pos, d: int, base: float) -> np.ndarray:
    """p * theta_i as float64, shape pos.shape + (d/2,)."""
    p = np.asarray(pos, dtype=np.float64)
    return p[..., None] * inv_freq(d, base)


def rotate(x, pos, base: float) -> np.ndarray:
    """Apply R(pos) to the last axis of x (float64).

    ``pos`` broadcasts against ``x.shape[:-1]``.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    a = angles(pos, d, base)
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def rotation_matrix(pos: float, d: int, base: float) -> np.ndarray:
    """The d x d matrix of R(pos) (for identity checks)."""
    return rotate(np.eye(d), np.full(d, pos), base).T
