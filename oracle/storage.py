"""Storage-faithful simulation of the rolling cache (oracle).

Same steps as the method, in float64, but every value the method STORES is
rounded the way it is stored: K and V live in bfloat16, so K is rounded to
bfloat16 (RNE) when it is appended with its rotation baked in (voxtral.c
explainer, section 二: RoPE is applied when K is written, so compaction never
re-encodes K) and again each time re-basing rewrites it in place (Audio8
explainer, "Rolling KV Cache 三步拆解", step 2).  Everything else (the query
rotation, scores, softmax, the weighted sum) is float64.

Compensated re-basing (a reading of "exact rotation" for bfloat16 storage):
a second bfloat16 array ``lo`` keeps the rounding residual of K, so the value
carried from one re-base to the next is hi + lo (about 16 significant bits)
instead of hi alone.  Attention reads hi only.

With ``rounder=None`` (no rounding) the simulation must reproduce the exact
oracle in :mod:`oracle.attention`; with bfloat16 rounding it predicts what a
correct bf16 implementation stores.  V is stored in the same format: with the
fp16 cache variant (``rounder=fp16.round_f16``; voxtral.c explainer, section
七, fp16 KV cache) the bfloat16 inputs are rounded to fp16 on append; with
bfloat16 storage that rounding is the identity.
"""
from __future__ import annotations

import math

import numpy as np

from . import rope
from . import schedule as sch
from .bf16 import round_bf16


def _identity(x):
    return np.asarray(x, np.float64)


def _store(rounder, v):
    """A V row as stored (rounded to the storage format, if any)."""
    return (rounder or _identity)(v)


def append_k(k_new, pos, base, compensated=False, rounder=round_bf16):
    """K row as stored on append: hi = rne(R(pos) k) and lo = rne(R(pos) k - hi)."""
    rounder = rounder or _identity
    y = rope.rotate(k_new, pos, base)
    hi = rounder(y)
    lo = rounder(y - hi) if compensated else np.zeros_like(hi)
    return hi, lo


def rebase_k(hi, lo, delta, base, compensated=False, rounder=round_bf16):
    """One in-place re-base of stored K rows by R(-delta).

    Plain: x = hi, hi' = rne(R(-delta) x).
    Compensated: x = hi + lo, hi' = rne(y), lo' = rne(y - hi') with y = R(-delta) x.
    """
    rounder = rounder or _identity
    x = np.asarray(hi, np.float64) + (np.asarray(lo, np.float64) if compensated else 0.0)
    y = rope.rotate(x, -float(delta), base)
    new_hi = rounder(y)
    new_lo = rounder(y - new_hi) if compensated else np.zeros_like(new_hi)
    return new_hi, new_lo


def _attend_rows(q_rot, k_rows, v_rows, group, scale, mask=None):
    """q_rot [nq, d] against k_rows/v_rows [n, d] (one KV head)."""
    out = np.empty_like(q_rot)
    for h in range(q_rot.shape[0]):
        s = (k_rows @ q_rot[h]) * scale
        if mask is not None:
            s = np.where(mask[h], s, -np.inf)
        s = s - s.max()
        p = np.exp(s)
        p /= p.sum()
        out[h] = p @ v_rows
    return out


class RebaseRing:
    """One (stream, layer) of the re-base ring, simulated step by step."""

    def __init__(self, hq, hkv, d, window, dc, base, origin=0,
                 compensated=False, rounder=round_bf16, scale=None):
        self.hq, self.hkv, self.d = hq, hkv, d
        self.window, self.dc, self.base = window, dc, base
        self.comp = compensated
        self.rounder = rounder
        self.scale = 1.0 / math.sqrt(d) if scale is None else scale
        self.state = sch.init_state(sch.MODE_REBASE, window, window, origin, dc)
        self.k_hi = np.zeros((hkv, window, d))
        self.k_lo = np.zeros((hkv, window, d))
        self.v = np.zeros((hkv, window, d))

    def step(self, q, k_new, v_new):
        """q [Hq, d], k_new/v_new [Hkv, d] raw inputs -> (plan, out[Hq, d])."""
        plan = sch.step(sch.MODE_REBASE, self.state, self.dc)
        n = plan.n_valid
        if plan.rebase_delta:
            rows = [r for r in range(n) if r != plan.slot]
            for g in range(self.hkv):
                hi, lo = rebase_k(self.k_hi[g, rows], self.k_lo[g, rows],
                                  plan.rebase_delta, self.base, self.comp, self.rounder)
                self.k_hi[g, rows], self.k_lo[g, rows] = hi, lo
        hi, lo = append_k(k_new, plan.pos, self.base, self.comp, self.rounder)
        self.k_hi[:, plan.slot] = hi
        self.k_lo[:, plan.slot] = lo
        self.v[:, plan.slot] = _store(self.rounder, v_new)
        q_rot = rope.rotate(q, plan.pos, self.base)
        group = self.hq // self.hkv
        out = np.empty((self.hq, self.d))
        for g in range(self.hkv):
            out[g * group:(g + 1) * group] = _attend_rows(
                q_rot[g * group:(g + 1) * group], self.k_hi[g, :n], self.v[g, :n],
                group, self.scale)
        return plan, out


class CompactBuffer:
    """One (stream, layer) of the compaction-mode buffer, simulated step by step."""

    def __init__(self, hq, hkv, d, window, cap, base, origin=0,
                 rounder=round_bf16, scale=None):
        self.hq, self.hkv, self.d = hq, hkv, d
        self.window, self.cap, self.base = window, cap, base
        self.rounder = rounder
        self.scale = 1.0 / math.sqrt(d) if scale is None else scale
        self.state = sch.init_state(sch.MODE_COMPACT, window, cap, origin)
        self.k = np.zeros((hkv, cap, d))
        self.v = np.zeros((hkv, cap, d))

    def step(self, q, k_new, v_new):
        plan = sch.step(sch.MODE_COMPACT, self.state)
        if plan.compact_drop:
            D = plan.compact_drop
            keep = self.window
            # the newest `keep` rows move to the front, in order (memmove)
            self.k[:, :keep] = self.k[:, D:D + keep].copy()
            self.v[:, :keep] = self.v[:, D:D + keep].copy()
        hi, _ = append_k(k_new, plan.pos, self.base, False, self.rounder)
        self.k[:, plan.slot] = hi
        self.v[:, plan.slot] = _store(self.rounder, v_new)
        n = plan.n_valid
        q_rot = rope.rotate(q, plan.pos, self.base)
        group = self.hq // self.hkv
        out = np.empty((self.hq, self.d))
        for g in range(self.hkv):
            out[g * group:(g + 1) * group] = _attend_rows(
                q_rot[g * group:(g + 1) * group], self.k[g, :n], self.v[g, :n],
                group, self.scale)
        return plan, out


class EncoderRing:
    """One (stream, layer) of the encoder chunk ring (multi-head)."""

    def __init__(self, heads, d, window, frames, base, origin=0, cap=None,
                 rounder=round_bf16, scale=None):
        self.h, self.d, self.window, self.f, self.base = heads, d, window, frames, base
        self.cap = window + frames if cap is None else cap
        self.origin = origin
        self.rounder = rounder
        self.scale = 1.0 / math.sqrt(d) if scale is None else scale
        self.state = sch.init_state(sch.MODE_ENC, window, self.cap, origin, 1, frames)
        self.k = np.zeros((heads, self.cap, d))
        self.v = np.zeros((heads, self.cap, d))

    def step(self, q, k_new, v_new):
        """q, k_new, v_new [F, H, d] raw -> (plan, out[F, H, d])."""
        plan = sch.step(sch.MODE_ENC, self.state, 1, self.f)
        for j in range(self.f):
            slot = (plan.slot + j) % self.cap
            hi, _ = append_k(k_new[j], plan.pos + j, self.base, False, self.rounder)
            self.k[:, slot] = hi
            self.v[:, slot] = v_new[j]
        slot_pos = sch.enc_slot_positions(plan, self.origin)
        written = np.array([p is not None for p in slot_pos])
        pos = np.array([-1 if p is None else p for p in slot_pos], np.int64)
        # every head and frame at once: s[h, r, j] = K[h, r] . R(pos + j) q[j, h]
        q_rot = np.stack([rope.rotate(q[j], plan.pos + j, self.base) for j in range(self.f)])
        s = np.matmul(self.k, q_rot.transpose(1, 2, 0)) * self.scale
        qpos = plan.pos + np.arange(self.f)
        vis = (written & (pos >= plan.first_pos))[:, None] & (pos[:, None] <= qpos[None, :])
        s = np.where(vis[None], s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out = np.matmul(p.transpose(0, 2, 1), self.v).transpose(1, 0, 2)     # [F, H, d]
        return plan, np.ascontiguousarray(out)
