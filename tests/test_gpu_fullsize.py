"""Full-size workloads in the launch configuration bench.py times (one
rkv_decode_step_pipelined launch per step over all layers, plans alternating
between two buffers; for the mixed-window workload also its default update
path, rkv_update_step + rkv_decode_attn_pipelined; rkv_encoder_chunk_attn
for the encoder; the same input pools), checked on sampled (layer, stream)
outputs that the oracle computes one by one, plus properties that hold at any
size (every plan bit-exact against the oracle schedule, all outputs
finite)."""
import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import fp16 as of
from oracle import schedule as sch
from oracle import storage as stg
from rolling_window_kv_amd import synth

from gpu_util import check_close, device, f64, rkv_mod, say

pytestmark = pytest.mark.gpu

HQ, HKV, D = 16, 2, 128


def _history(pool_pair, steps):
    """Inputs of steps 0..steps-1 of one pair from its pool (entry t % P)."""
    q, k, v = pool_pair
    idx = np.arange(steps) % q.shape[0]
    return tuple(f64(x)[idx] for x in (q, k, v))


def _check_plans(rkv, got, mode, windows, caps, origins, steps, dc=1, F=1):
    """got: the plans (PLAN_DTYPE) of step steps - 1."""
    S = len(windows)
    for s in range(S):
        st = sch.init_state(mode, int(windows[s]), int(caps[s]), int(origins[s]), dc, F)
        for _ in range(steps):
            ref = sch.step(mode, st, dc, F)
        for f in ("t", "pos", "pos_offset", "first_pos", "slot", "n_valid", "rebase_delta",
                  "compact_drop", "evict_slot", "evict_pos"):
            assert int(got[f][s]) == getattr(ref, f), (s, f)


def _run_decoder_bench(rkv, cfg, slots, windows, caps, origins, q, k, v, steps, keep=(),
                       path="pipelined"):
    """The bench's step: rkv_advance primes the first plan, then per step (after
    rkv_compact in compaction mode) one pipelined launch (pipelined), or
    rkv_update_step + rkv_decode_attn_pipelined (update), plans alternating
    between two buffers.  Returns the cache, the last output, kept outputs
    and the last step's plans."""
    dev = q.device
    P = q.shape[0]
    cache = rkv.Cache(cfg, slots, windows, caps, origins, device=dev, zero=False)
    out = torch.empty(q.shape[1:], dtype=torch.bfloat16, device=dev)
    plans = [cache.plan, cache.plan_next]
    rkv.rkv_advance(cfg, cache.state, plans[0])
    kept = {}
    for t in range(steps):
        j = t % P
        cur, nxt = plans[t % 2], plans[(t + 1) % 2]
        if cfg.mode == rkv.RKV_MODE_COMPACT:
            rkv.rkv_compact(cfg, cur, cache.kv)
        if path == "update":
            rkv.rkv_update_step(cfg, cur, cache.kv, k[j], v[j])
            rkv.rkv_decode_attn_pipelined(cfg, cache.state, cur, nxt, cache.kv, q[j], out,
                                          cache.workspace)
        else:
            rkv.rkv_decode_step_pipelined(cfg, cache.state, cur, nxt, cache.kv, q[j], k[j], v[j],
                                          out, cache.workspace)
        if t in keep:
            kept[t] = out.clone()
    torch.cuda.synchronize()
    last = plans[(steps - 1) % 2].cpu().numpy().view(rkv.PLAN_DTYPE)
    return cache, out, kept, last


@pytest.mark.parametrize("fp16", [False, True])
def test_decode_36_layers_64_streams_w375(fp16):
    rkv = rkv_mod()
    dev = device()
    L, S, W, dc, P, seed = 36, 64, 375, 25, 64, 1002
    steps = 450                                         # fills, then re-bases at 399, 424, 449
    q, k, v = synth.decoder_pool(seed, L, S, P, HQ, HKV, D)
    cfg = rkv.make_cfg(S, L, rebase_chunk=dc, flags=rkv.RKV_F_KV_FP16 if fp16 else 0)
    say(f"case: 36x64 W=375 dc=25, 450 pipelined steps, fp16 cache {fp16}")
    cache, out, kept, last = _run_decoder_bench(rkv, cfg, W, W, W, 0, q.to(dev), k.to(dev),
                                                v.to(dev), steps, keep=(420,))
    assert torch.isfinite(out.float()).all()
    _check_plans(rkv, last, sch.MODE_REBASE, [W] * S, [W] * S, [0] * S, steps, dc)
    got = {449: f64(out), 420: f64(kept[420])}
    for (l, s) in [(0, 0), (35, 63), (17, 5), (3, 40), (29, 22)]:
        pair = synth.decoder_pair(seed, l, s, P, HQ, HKV, D)
        qh, kh, vh = _history(pair, steps)
        exact = att.window_decode(qh, kh, vh, W, 1e6, steps=[420, 449])
        ring = stg.RebaseRing(HQ, HKV, D, W, dc, 1e6,
                              rounder=of.round_f16 if fp16 else stg.round_bf16)
        sf = {t: ring.step(qh[t], kh[t], vh[t])[1] for t in range(steps)}
        for t in (420, 449):
            check_close(got[t][l, s], exact[t], 2e-2, f"36x64 l{l} s{s} t{t} vs exact")
            check_close(got[t][l, s], sf[t], 1e-3, f"36x64 l{l} s{s} t{t} vs storage-faithful",
                        ulp_slack=True)


@pytest.mark.parametrize("path", ["update", "pipelined"])
def test_decode_mixed_clocks_256_streams_outliers(path):
    rkv = rkv_mod()
    dev = device()
    L, S, dc, P, seed = 36, 256, 25, 16, 1003
    windows = np.repeat(np.array([375, 250, 188], np.int32), [86, 85, 85])
    t0 = synth.start_offsets(seed, S, 5000)
    origins = np.maximum(0, t0 - windows).astype(np.int64)
    steps = 375 + 60
    q, k, v = synth.decoder_pool(seed, L, S, P, HQ, HKV, D, 0.01)
    cfg = rkv.make_cfg(S, L, rebase_chunk=dc)
    say(f"case: 36x256 mixed W, offsets, outliers, {path} path")
    cache, out, _, last = _run_decoder_bench(rkv, cfg, 375, windows, windows, origins,
                                             q.to(dev), k.to(dev), v.to(dev), steps, path=path)
    assert torch.isfinite(out.float()).all()
    _check_plans(rkv, last, sch.MODE_REBASE, windows, windows, origins, steps, dc)
    got = f64(out)
    T = steps - 1
    for (l, s) in [(0, 0), (20, 85), (35, 86), (7, 170), (30, 171), (11, 255)]:
        pair = synth.decoder_pair(seed, l, s, P, HQ, HKV, D, 0.01)
        qh, kh, vh = _history(pair, steps)
        W, o = int(windows[s]), int(origins[s])
        ring = stg.RebaseRing(HQ, HKV, D, W, dc, 1e6, origin=o)
        for t in range(steps):
            _, sf = ring.step(qh[t], kh[t], vh[t])
        check_close(got[l, s], sf, 2e-2, f"mixed l{l} s{s} W{W} vs storage-faithful",
                    ulp_slack=True)
        exact = att.window_decode(qh, kh, vh, W, 1e6, origin=o, steps=[T])[T]
        err = np.abs(got[l, s] - exact)
        say(f"  info: vs exact max {err.max():.3e}, above 2e-2: {float((err > 2e-2).mean()):.4%}")


def test_compaction_26_layers_16_streams_w8192():
    rkv = rkv_mod()
    dev = device()
    L, S, W, cap, P, seed = 26, 16, 8192, 9216, 16, 1004
    steps = cap + 30                                    # first compaction at step 9216
    q, k, v = synth.decoder_pool(seed, L, S, P, HQ, HKV, D)
    cfg = rkv.make_cfg(S, L, mode=rkv.RKV_MODE_COMPACT)
    say("case: 26x16 W=8192 cap=9216 compaction")
    cache, out, _, last = _run_decoder_bench(rkv, cfg, cap, W, cap, 0, q.to(dev), k.to(dev),
                                             v.to(dev), steps)
    assert torch.isfinite(out.float()).all()
    _check_plans(rkv, last, sch.MODE_COMPACT, [W] * S, [cap] * S, [0] * S, steps)
    got = f64(out)
    T = steps - 1
    for (l, s) in [(0, 0), (25, 15), (13, 7)]:
        pair = synth.decoder_pair(seed, l, s, P, HQ, HKV, D)
        qh, kh, vh = _history(pair, steps)
        exact = att.compact_decode(qh, kh, vh, W, cap, 1e6, steps=[T])[T]
        check_close(got[l, s], exact, 2e-2, f"compact l{l} s{s} vs exact")


def test_encoder_32_layers_128_streams():
    rkv = rkv_mod()
    dev = device()
    L, S, H, d, F, W, P, seed = 32, 128, 20, 64, 4, 750, 4, 1005
    cap = W + F
    steps = 200                                          # the 754-slot ring wraps at step 189
    q, k, v = synth.encoder_pool(seed, L, S, P, F, H, d)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    cfg = rkv.make_cfg(S, L, num_q_heads=H, num_kv_heads=H, head_dim=d,
                       mode=rkv.RKV_MODE_ENC_CHUNK, new_rows=F)
    say("case: encoder 32x128 H=20 d=64 F=4 W=750")
    cache = rkv.Cache(cfg, cap, W, cap, 0, device=dev, zero=False)
    out = torch.empty(q.shape[1:], dtype=torch.bfloat16, device=dev)
    for t in range(steps):
        rkv.rkv_advance(cfg, cache.state, cache.plan)
        rkv.rkv_encoder_chunk_attn(cfg, cache.plan, cache.kv, qd[t % P], kd[t % P], vd[t % P],
                                   out, cache.workspace)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    _check_plans(rkv, cache.plan_host(), sch.MODE_ENC, [W] * S, [cap] * S, [0] * S, steps, 1, F)
    got = f64(out)
    for (l, s) in [(0, 0), (31, 127), (16, 64)]:
        pair = synth.encoder_pair(seed, l, s, P, F, H, d)
        qh, kh, vh = _history(pair, steps)
        exact = att.encoder_chunks(qh, kh, vh, W, 1e6, chunks=[steps - 1])[steps - 1]
        check_close(got[l, s], exact, 2e-2, f"encoder l{l} s{s} vs exact")
