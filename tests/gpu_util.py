"""Shared drivers for the GPU parity tests (everything goes through the C ABI)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle.bf16 import bf16_ulp


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def rkv_mod():
    from rolling_window_kv_amd import rkv
    rkv.lib()          # raises if the library is missing: no fallback
    return rkv


def f64(t):
    return t.detach().float().cpu().double().numpy()


def say(*a):
    print(*a, flush=True)


def run_decoder(rkv, cfg, slots, windows, caps, origins, q, k, v, fused, steps=None,
                keep_plans=False, out_dtype=torch.bfloat16):
    """Drive REBASE or COMPACT mode for ``steps`` steps on device inputs.

    q: [T, L, S, Hq, d], k/v: [T, L, S, Hkv, d] bf16 device tensors (step t
    reads entry t % T).  Returns (cache, out[steps, L, S, Hq, d], plans or None).
    """
    dev = q.device
    T = q.shape[0]
    steps = T if steps is None else steps
    cache = rkv.Cache(cfg, slots, windows, caps, origins, device=dev)
    out = torch.zeros((steps,) + tuple(q.shape[1:]), dtype=out_dtype, device=dev)
    plans = []
    for t in range(steps):
        i = t % T
        rkv.rkv_advance(cfg, cache.state, cache.plan)
        if cfg.mode == rkv.RKV_MODE_COMPACT:
            rkv.rkv_compact(cfg, cache.plan, cache.kv)
        if fused:
            rkv.rkv_decode_step(cfg, cache.plan, cache.kv, q[i], k[i], v[i], out[t],
                                cache.workspace)
        else:
            if cfg.mode == rkv.RKV_MODE_REBASE:
                rkv.rkv_roll_rebase(cfg, cache.plan, cache.kv)
            rkv.rkv_append(cfg, cache.plan, cache.kv, k[i], v[i])
            rkv.rkv_decode_attn(cfg, cache.plan, cache.kv, q[i], out[t], cache.workspace)
        if keep_plans:
            plans.append(cache.plan.clone())
    torch.cuda.synchronize()
    if keep_plans:
        plans = [p.cpu().numpy().view(rkv.PLAN_DTYPE) for p in plans]
    return cache, out, (plans if keep_plans else None)


def run_encoder(rkv, cfg, slots, windows, caps, origins, q, k, v, steps=None):
    """Drive ENC_CHUNK mode; q/k/v: [T, L, S, F, H, d] bf16 device tensors."""
    dev = q.device
    T = q.shape[0]
    steps = T if steps is None else steps
    cache = rkv.Cache(cfg, slots, windows, caps, origins, device=dev)
    out = torch.zeros((steps,) + tuple(q.shape[1:]), dtype=torch.bfloat16, device=dev)
    for t in range(steps):
        i = t % T
        rkv.rkv_advance(cfg, cache.state, cache.plan)
        rkv.rkv_encoder_chunk_attn(cfg, cache.plan, cache.kv, q[i], k[i], v[i], out[t],
                                   cache.workspace)
    torch.cuda.synchronize()
    return cache, out


def check_close(got, want, atol, label, ulp_slack=False):
    """max |got - want| <= atol (+ one bf16 ulp of want when ulp_slack)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want)
    tol = atol + (bf16_ulp(want) if ulp_slack else 0.0)
    bad = err > tol
    say(f"{label}: max|err| {err.max():.3e} (tol {atol:g}{' + 1 ulp' if ulp_slack else ''}),"
        f" violations {int(bad.sum())}")
    assert not bad.any(), f"{label}: {int(bad.sum())} elements above tolerance, max {err.max()}"
    return float(err.max())
