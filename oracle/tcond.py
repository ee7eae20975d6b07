"""Delay conditioning t_cond (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring): float64 NumPy.

Audio8 ASR Infinite explainer, 可配置转写延迟: the model is told how many
clock steps it runs behind real time, num_delay_tokens = target_delay_ms /
clock (480 ms at the 80 ms clock gives 6).  That count is turned into a
sinusoidal time embedding, a frame-length embedding is added, and the sum,
the condition vector t_cond, modulates the decoder's hidden state after the
attention of every layer.  Model card, 优化操作点: target_delay_ms must be an
integer multiple of the selected clock; the clocks are 80 / 120 / 160 ms
(frame_len 4 / 6 / 8 tower frames of 20 ms).  Model card, 架构: the
frame-length embedding is a trained component (random initialisation).

Readings taken where the pages give no detail (the form of the modulation is
not given, so parity of that form is unpinned; the steps below are pinned
against hand-worked values and identities):

  * sinusoidal embedding of even width D: e_i = sin(n w_i), e_{D/2+i} =
    cos(n w_i), w_i = 10000^(-i / (D/2)), i < D/2 -- the transformer's
    sinusoidal code with the delay count n as the position;
  * the frame-length embedding is one table row per frame_len;
    t_cond = e(n) + table[frame_len];
  * the modulation after the attention of layer l is a feature-wise scale
    and shift: h <- h * (1 + gamma_l) + beta_l, [gamma_l; beta_l] = A_l t_cond
    with A_l of shape [2 H, D] (no bias), H = the hidden width;
  * h is the layer's attention output (16 heads x 128 = 2048 features, the
    decoder's hidden width), stored as bfloat16 after the modulation.
"""
from __future__ import annotations

import numpy as np

from .bf16 import round_bf16

CLOCKS_MS = (80, 120, 160)
TOWER_FRAME_MS = 20
BASE = 10000.0


def delay_tokens(target_delay_ms: int, clock_ms: int):
    """(num_delay_tokens, frame_len) for a delay and an audio clock; ValueError
    for a clock other than 80 / 120 / 160 ms or a delay that is not a positive
    integer multiple of it."""
    if clock_ms not in CLOCKS_MS:
        raise ValueError(f"clock {clock_ms} ms is not one of {CLOCKS_MS}")
    if target_delay_ms <= 0 or target_delay_ms % clock_ms:
        raise ValueError(f"delay {target_delay_ms} ms is not a multiple of the {clock_ms} ms clock")
    return target_delay_ms // clock_ms, clock_ms // TOWER_FRAME_MS


def sinusoid(n, dim: int) -> np.ndarray:
    """[dim] sinusoidal embedding of the count n (sines first, then cosines)."""
    if dim % 2:
        raise ValueError("dim must be even")
    half = dim // 2
    w = BASE ** (-np.arange(half, dtype=np.float64) / half)
    a = float(n) * w
    return np.concatenate([np.sin(a), np.cos(a)])


def t_cond(n, frame_len: int, frame_table) -> np.ndarray:
    table = np.asarray(frame_table, np.float64)
    return sinusoid(n, table.shape[1]) + table[frame_len]


def modulation(A, tc):
    """A [2H, D], t_cond [D] -> (gamma [H], beta [H])."""
    m = np.asarray(A, np.float64) @ np.asarray(tc, np.float64)
    H = m.shape[0] // 2
    return m[:H], m[H:]


def modulate(h, gamma, beta, rounder=round_bf16):
    """Feature-wise scale and shift of the hidden state h [..., H]."""
    r = rounder or (lambda x: np.asarray(x, np.float64))
    return r(np.asarray(h, np.float64) * (1.0 + gamma) + beta)
