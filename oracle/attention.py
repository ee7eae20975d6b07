"""Exact attention over the rolling window (oracle).

"Exact" means: the raw (un-rotated) q/k/v history is kept, RoPE is applied at
each token's absolute (or logical) position in float64, and nothing is rounded
in between.  This is the result the rolling cache must reproduce, since RoPE
attention scores depend only on position differences: re-basing (Audio8
explainer, "Rolling KV Cache 三步拆解", step 2) and the logical-offset
compaction (voxtral.c explainer, section 二) are both meant to leave it
unchanged.

Readings where the pages are silent: softmax scale 1/sqrt(d), no attention
sinks and no soft-capping; the new token is appended before it attends, so it
sees itself; query head h reads KV head h // (Hq / Hkv) (grouped-query
attention, 16 query heads over 2 KV heads on the Audio8 decoder, model card
"架构" checkpoint specification).
"""
from __future__ import annotations

import math

import numpy as np

from . import rope
from . import schedule as sch


def softmax_attend(q_rot, k_rot, v, scale):
    """One query block against one key block, float64.

    q_rot [Hq, d], k_rot [n, Hkv, d], v [n, Hkv, d] -> [Hq, d].
    """
    hq = q_rot.shape[0]
    hkv = k_rot.shape[1]
    group = hq // hkv
    out = np.empty_like(q_rot)
    for h in range(hq):
        g = h // group
        s = (k_rot[:, g, :] @ q_rot[h]) * scale
        s = s - s.max()
        p = np.exp(s)
        p /= p.sum()
        out[h] = p @ v[:, g, :]
    return out


def attend_history(q_hist, k_hist, v_hist, first_idx, base, origin=0,
                   scale=None, steps=None):
    """Decode outputs for steps ``steps`` of one (stream, layer).

    q_hist [T, Hq, d], k_hist/v_hist [T, Hkv, d]: raw inputs of positions
    origin .. origin+T-1.  ``first_idx[i]`` is the history index of the oldest
    key that step i attends to; keys first_idx[i] .. i are attended.
    Returns {i: out[Hq, d]} (float64).
    """
    q_hist = np.asarray(q_hist, np.float64)
    k_hist = np.asarray(k_hist, np.float64)
    v_hist = np.asarray(v_hist, np.float64)
    T, _, d = q_hist.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if steps is None:
        steps = range(T)
    pos = origin + np.arange(T)
    k_rot = rope.rotate(k_hist, pos[:, None], base)
    out = {}
    for i in steps:
        q_rot = rope.rotate(q_hist[i], np.full(q_hist.shape[1], origin + i), base)
        lo = first_idx[i]
        out[i] = softmax_attend(q_rot, k_rot[lo:i + 1], v_hist[lo:i + 1], scale)
    return out


def window_decode(q_hist, k_hist, v_hist, window, base, origin=0, scale=None,
                  steps=None):
    """Rolling-window decode: step i attends to the last ``window`` tokens."""
    T = np.asarray(q_hist).shape[0]
    first = [max(0, i - window + 1) for i in range(T)]
    return attend_history(q_hist, k_hist, v_hist, first, base, origin, scale, steps)


def compact_decode(q_hist, k_hist, v_hist, window, cap, base, origin=0,
                   scale=None, steps=None):
    """Compaction-mode decode: step i attends to every retained row.

    The retained rows are logical positions [kv_pos_offset, t], taken from the
    compaction schedule.
    """
    T = np.asarray(q_hist).shape[0]
    plans = sch.run(sch.MODE_COMPACT, T, window, cap, origin)
    first = [p.first_pos - origin for p in plans]
    return attend_history(q_hist, k_hist, v_hist, first, base, origin, scale, steps)


def encoder_chunks(q, k, v, window, base, origin=0, scale=None, chunks=None):
    """Encoder chunk attention (multi-head, every head has its own K/V).

    q, k, v: [n_chunks, F, H, d] raw inputs; chunk n holds frames at logical
    positions P + j with P = origin + n F.  Frame j attends to positions
    [max(origin, P - window), P + j].  Returns {n: out[F, H, d]}.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n_chunks, F, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if chunks is None:
        chunks = range(n_chunks)
    frames_k = k.reshape(n_chunks * F, H, d)
    frames_v = v.reshape(n_chunks * F, H, d)
    pos = origin + np.arange(n_chunks * F)
    k_rot = rope.rotate(frames_k, pos[:, None], base)
    out = {}
    for n in chunks:
        P = origin + n * F
        res = np.empty((F, H, d))
        for j in range(F):
            lo = max(origin, P - window) - origin
            hi = P + j - origin
            q_rot = rope.rotate(q[n, j], np.full(H, P + j), base)
            for h in range(H):
                s = (k_rot[lo:hi + 1, h, :] @ q_rot[h]) * scale
                s = s - s.max()
                p = np.exp(s)
                p /= p.sum()
                res[j, h] = p @ frames_v[lo:hi + 1, h, :]
        out[n] = res
    return out
