"""Seeded synthetic inputs (q, k_new, v_new) for the rolling-KV workloads.

This module only draws random numbers; it holds none of the method's
arithmetic, so both the GPU path's tests/benchmark and the CPU oracle consume
exactly the same bfloat16 values from it.

Every (layer, stream) pair owns an independent NumPy generator seeded with
``[seed, layer, stream]``, so any pair's inputs can be regenerated on its own.
A step pool of ``period`` entries is drawn per pair; step i uses entry
``i % period`` (the benchmark cycles a device-resident pool; parity runs use a
period at least as long as the run so no entry repeats).

Values are N(0, 1) in float32, optionally with element-wise outliers
(probability ``outlier_frac``, scaled by ``outlier_scale``), then rounded to
bfloat16 by torch (round to nearest even).
"""
from __future__ import annotations

import numpy as np
import torch


def _block(seed, layer, stream, shape, outlier_frac=0.0, outlier_scale=8.0):
    rng = np.random.default_rng([int(seed), int(layer), int(stream)])
    x = rng.standard_normal(shape, dtype=np.float32)
    if outlier_frac > 0.0:
        hit = rng.random(shape, dtype=np.float32) < outlier_frac
        x = np.where(hit, x * np.float32(outlier_scale), x)
    return x


def decoder_pair(seed, layer, stream, period, hq, hkv, d, outlier_frac=0.0):
    """One (layer, stream): q [P, Hq, d], k [P, Hkv, d], v [P, Hkv, d] (bf16, CPU)."""
    x = _block(seed, layer, stream, (period, hq + 2 * hkv, d), outlier_frac)
    t = torch.from_numpy(x).to(torch.bfloat16)
    return t[:, :hq].contiguous(), t[:, hq:hq + hkv].contiguous(), t[:, hq + hkv:].contiguous()


def decoder_pool(seed, layers, streams, period, hq, hkv, d, outlier_frac=0.0):
    """All pairs: q [P, L, S, Hq, d], k/v [P, L, S, Hkv, d] (bf16, CPU).

    ``layers``/``streams`` are counts; pair (l, s) equals
    ``decoder_pair(seed, l, s, ...)``.
    """
    q = torch.empty((period, layers, streams, hq, d), dtype=torch.bfloat16)
    k = torch.empty((period, layers, streams, hkv, d), dtype=torch.bfloat16)
    v = torch.empty((period, layers, streams, hkv, d), dtype=torch.bfloat16)
    for l in range(layers):
        for s in range(streams):
            q[:, l, s], k[:, l, s], v[:, l, s] = decoder_pair(
                seed, l, s, period, hq, hkv, d, outlier_frac)
    return q, k, v


def encoder_pair(seed, layer, stream, period, frames, heads, d):
    """One (layer, stream): q, k, v each [P, F, H, d] (bf16, CPU)."""
    x = _block(seed, layer, stream, (period, 3, frames, heads, d))
    t = torch.from_numpy(x).to(torch.bfloat16)
    return t[:, 0].contiguous(), t[:, 1].contiguous(), t[:, 2].contiguous()


def encoder_pool(seed, layers, streams, period, frames, heads, d):
    """All pairs: q, k, v each [P, L, S, F, H, d] (bf16, CPU)."""
    shape = (period, layers, streams, frames, heads, d)
    q, k, v = (torch.empty(shape, dtype=torch.bfloat16) for _ in range(3))
    for l in range(layers):
        for s in range(streams):
            q[:, l, s], k[:, l, s], v[:, l, s] = encoder_pair(
                seed, l, s, period, frames, heads, d)
    return q, k, v


def start_offsets(seed, streams, high):
    """Per-stream start offsets, uniform integers in [0, high]."""
    rng = np.random.default_rng([int(seed), 0x5EED])
    return rng.integers(0, high + 1, size=streams).astype(np.int64)


def encoder_stack_weights(seed, layers, hidden, ffn):
    """Synthetic weights of a stack of pre-norm encoder layers (CPU bf16).

    Per layer a dict: g1, g2 [hidden] = 1 + 0.1 N(0, 1); wq, wk, wv, wo
    [hidden, hidden] and w1 [ffn, hidden], w2 [hidden, ffn] = N(0, 1) /
    sqrt(fan_in) (row = output feature).  Layer l draws from [seed, l, -1].
    """
    out = []
    for l in range(layers):
        rng = np.random.default_rng([int(seed), int(l), 2 ** 31 - 1])

        def mat(rows, cols):
            x = rng.standard_normal((rows, cols), dtype=np.float32) / np.float32(np.sqrt(cols))
            return torch.from_numpy(x).to(torch.bfloat16)

        def gain():
            x = 1.0 + 0.1 * rng.standard_normal(hidden, dtype=np.float32)
            return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)

        out.append(dict(g1=gain(), wq=mat(hidden, hidden), wk=mat(hidden, hidden),
                        wv=mat(hidden, hidden), wo=mat(hidden, hidden), g2=gain(),
                        w1=mat(ffn, hidden), w2=mat(hidden, ffn)))
    return out


def encoder_stack_inputs(seed, streams, period, frames, hidden):
    """Frame embeddings entering the stack: [period, S, F, hidden] float32 N(0, 1)."""
    rng = np.random.default_rng([int(seed), 2 ** 31 - 2])
    return torch.from_numpy(rng.standard_normal((period, streams, frames, hidden),
                                                dtype=np.float32))


def tcond_weights(seed, layers, hidden, dim, max_frame_len=8):
    """Synthetic delay-conditioning weights (CPU bf16): the frame-length table
    [max_frame_len + 1, dim] = N(0, 1) and per layer the modulation matrix
    [layers, 2 hidden, dim] = 0.1 N(0, 1) / sqrt(dim) (rows: scale, then shift)."""
    rng = np.random.default_rng([int(seed), 2 ** 31 - 3])
    table = rng.standard_normal((max_frame_len + 1, dim), dtype=np.float32)
    A = rng.standard_normal((layers, 2 * hidden, dim), dtype=np.float32) * np.float32(
        0.1 / np.sqrt(dim))
    return (torch.from_numpy(table).to(torch.bfloat16), torch.from_numpy(A).to(torch.bfloat16))
