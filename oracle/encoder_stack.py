"""Incremental encoder step through a stack of layers (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring): float64 NumPy.

voxtral.c explainer, section 三: the causal audio encoder (32 layers; the
Audio8 explainer's table: hidden 1280, a 750-frame sliding window) encodes
only the new positions of each step, each layer attending from the new
frames to its cached K/V.  This runs that step through every layer with the
chunk attention of :class:`oracle.storage.EncoderRing` (K rotated at its
logical position and rounded to bfloat16 when stored).

Readings taken where the pages give no detail of the layer: a pre-norm
residual layer, x += Wo attn(RMSNorm(x) Wq, Wk, Wv); x += W2 gelu(W1
RMSNorm(x)), with RMSNorm(x) = x / sqrt(mean(x^2) + eps) * g, the exact
(erf) GELU, an MLP of 4 x hidden, no biases; 20 heads of 64 as the encoder's
chosen split.  Storage-faithful points (as the GPU stores them): the normed
activations, q, k, v, the attention output and the MLP activation are
bfloat16; the residual stream stays in full precision (float32 on the GPU).
"""
from __future__ import annotations

import math

import numpy as np
from scipy import special

from . import storage
from .bf16 import round_bf16


def rmsnorm(x, g, eps):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def gelu(x):
    """Exact GELU, 0.5 x (1 + erf(x / sqrt 2)) (erf to float64 accuracy)."""
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1.0 + special.erf(x / math.sqrt(2.0)))


class EncoderStack:
    """One stream's encoder layers, stepped F frames at a time."""

    def __init__(self, weights, heads, d, window, frames, base, eps, origin=0,
                 rounder=round_bf16):
        self.w = [{n: np.asarray(t, np.float64) for n, t in lw.items()} for lw in weights]
        self.h, self.d, self.f, self.eps = heads, d, frames, eps
        self.r = rounder or (lambda x: np.asarray(x, np.float64))
        self.rings = [storage.EncoderRing(heads, d, window, frames, base, origin,
                                          rounder=rounder) for _ in weights]

    def run(self, xs):
        """xs [T, F, hidden]: T consecutive steps -> the stack's outputs [T, F, hidden].

        The same values as T calls of step(), computed layer by layer: every
        map of a layer but the chunk attention acts on each frame's row alone,
        so a layer takes all T steps' rows at once and only its attention
        walks the steps in order (the ring holds the earlier steps' K/V)."""
        xs = np.asarray(xs, np.float64)
        T = xs.shape[0]
        r, F, H, d = self.r, self.f, self.h, self.d
        x = xs.reshape(T * F, -1).copy()
        for w, ring in zip(self.w, self.rings):
            a = r(rmsnorm(x, w["g1"], self.eps))
            q, k, v = (r(a @ w[n].T).reshape(T, F, H, d) for n in ("wq", "wk", "wv"))
            att = np.stack([ring.step(q[t], k[t], v[t])[1] for t in range(T)])
            x = x + r(att).reshape(T * F, H * d) @ w["wo"].T
            a2 = r(rmsnorm(x, w["g2"], self.eps))
            u = r(gelu(a2 @ w["w1"].T))
            x = x + u @ w["w2"].T
        return x.reshape(xs.shape)

    def step(self, x):
        """x [F, hidden] (the residual stream entering layer 0) -> after the last layer."""
        x = np.asarray(x, np.float64)
        r, F, H, d = self.r, self.f, self.h, self.d
        for w, ring in zip(self.w, self.rings):
            a = r(rmsnorm(x, w["g1"], self.eps))
            q, k, v = (r(a @ w[n].T).reshape(F, H, d) for n in ("wq", "wk", "wv"))
            _, att = ring.step(q, k, v)
            x = x + r(att).reshape(F, H * d) @ w["wo"].T
            a2 = r(rmsnorm(x, w["g2"], self.eps))
            u = r(gelu(a2 @ w["w1"].T))
            x = x + u @ w["w2"].T
        return x
