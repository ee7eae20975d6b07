"""Merging split key ranges inside the attention launch (the last split of an
item to finish merges, counted by a per-item counter in the workspace)
against the separate merge launch (RKV_F_MERGE_LAUNCH): outputs and rings
must be identical bit for bit, on every path that splits -- fused and
read-only decode, re-base every position with the residual, compaction, the
pipelined step, float32 output, encoder chunks -- with 2 to 12 splits (12:
the merge reads the partials in two batches of up to 8).  Outputs are filled
with NaN before every step, so a merge that never happened shows, and the
counters must be back at zero after every call.  The in-launch merge also
meets the storage-faithful oracle's gate on its own.  A launch of more than
768 workgroups (items x splits) merges in the second launch whatever the flag
says; that choice is checked the same way."""
import numpy as np
import pytest
import torch

from oracle import storage as stg

from gpu_util import check_close, device, f64, rkv_mod, say

pytestmark = pytest.mark.gpu

HQ, HKV, D = 16, 2, 128


def _pool(seed, shape_q, shape_kv, dev):
    gen = torch.Generator().manual_seed(seed)
    q = torch.randn(shape_q, generator=gen).to(torch.bfloat16)
    k = torch.randn(shape_kv, generator=gen).to(torch.bfloat16)
    v = torch.randn(shape_kv, generator=gen).to(torch.bfloat16)
    return q, k, v, q.to(dev), k.to(dev), v.to(dev)


def _items(cfg):
    return cfg.num_layers * cfg.num_streams * cfg.num_kv_heads


def _counters_zero(rkv, cfg, cache):
    n = _items(cfg)
    words = cache.workspace.view(torch.int32)[:n]
    assert int((words != 0).sum()) == 0, "merge counters not returned to zero"


def _run(rkv, cfg, slots, windows, caps, origins, q, k, v, path, steps, out_dtype):
    """Decoder steps on one of the paths; returns (cache, outputs)."""
    dev = q.device
    cache = rkv.Cache(cfg, slots, windows, caps, origins, device=dev)
    assert cache.workspace is not None, "case must split the key range"
    out = torch.full((steps,) + tuple(q.shape[1:]), float("nan"), dtype=out_dtype, device=dev)
    T = q.shape[0]
    plans = [cache.plan, cache.plan_next]
    if path == "pipelined":
        rkv.rkv_advance(cfg, cache.state, plans[0])
    for t in range(steps):
        i = t % T
        if path == "pipelined":
            cur, nxt = plans[t % 2], plans[(t + 1) % 2]
            if cfg.mode == rkv.RKV_MODE_COMPACT:
                rkv.rkv_compact(cfg, cur, cache.kv)
            rkv.rkv_decode_step_pipelined(cfg, cache.state, cur, nxt, cache.kv, q[i], k[i], v[i],
                                          out[t], cache.workspace)
            continue
        rkv.rkv_advance(cfg, cache.state, cache.plan)
        if cfg.mode == rkv.RKV_MODE_COMPACT:
            rkv.rkv_compact(cfg, cache.plan, cache.kv)
        if path == "fused":
            rkv.rkv_decode_step(cfg, cache.plan, cache.kv, q[i], k[i], v[i], out[t],
                                cache.workspace)
        else:
            rkv.rkv_update_step(cfg, cache.plan, cache.kv, k[i], v[i])
            rkv.rkv_decode_attn(cfg, cache.plan, cache.kv, q[i], out[t], cache.workspace)
    torch.cuda.synchronize()
    return cache, out


CASES = [
    # name, mode, L, S, W, cap, dc, flags, splits, path, steps
    ("rebase-2", "rebase", 2, 3, 200, 200, 7, 0, 2, "fused", 90),
    ("rebase-5-read", "rebase", 2, 3, 200, 200, 7, 0, 5, "read", 90),
    ("rebase-12", "rebase", 1, 2, 200, 200, 7, 0, 12, "fused", 60),
    ("comp-every-step", "rebase", 1, 1, 375, 375, 1, "comp", 0, "fused", 420),
    ("pipelined-3", "rebase", 2, 2, 120, 120, 5, 0, 3, "pipelined", 150),
    ("f32-out-4", "rebase", 1, 2, 100, 100, 3, "f32", 4, "fused", 130),
    ("compact-3", "compact", 2, 2, 64, 80, 1, 0, 3, "fused", 200),
    ("many-blocks-4", "rebase", 2, 100, 64, 64, 4, 0, 4, "fused", 80),   # 1600 blocks
]
ORACLE_STREAMS = 4      # streams per layer checked against the oracle


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_in_launch_merge_matches_merge_launch(case):
    name, mode, L, S, W, cap, dc, flags, splits, path, steps = case
    rkv = rkv_mod()
    dev = device()
    fl = {0: 0, "comp": rkv.RKV_F_COMPENSATED, "f32": rkv.RKV_F_OUT_F32}[flags]
    md = rkv.RKV_MODE_REBASE if mode == "rebase" else rkv.RKV_MODE_COMPACT
    out_dtype = torch.float32 if flags == "f32" else torch.bfloat16
    origins = np.arange(S, dtype=np.int64) * 13
    T = min(steps, 64)
    qc, kc, vc, q, k, v = _pool(4100 + len(name), (T, L, S, HQ, D), (T, L, S, HKV, D), dev)
    outs, rings = [], []
    for merge_flag in (0, rkv.RKV_F_MERGE_LAUNCH):
        cfg = rkv.make_cfg(S, L, mode=md, rebase_chunk=dc, flags=fl | merge_flag,
                           num_splits=splits)
        say(f"case {name}: L={L} S={S} W={W} cap={cap} dc={dc} splits="
            f"{splits or 'auto'} path={path} merge={'launch' if merge_flag else 'in-launch'}")
        cache, out = _run(rkv, cfg, cap, W, cap, origins, q, k, v, path, steps, out_dtype)
        if not merge_flag:
            _counters_zero(rkv, cfg, cache)
        outs.append(out)
        rings.append(cache.buf)
    assert bool(torch.isfinite(outs[0].float()).all()), "an output was never written"
    ia = outs[0].view(torch.int32 if out_dtype == torch.float32 else torch.int16)
    ib = outs[1].view(torch.int32 if out_dtype == torch.float32 else torch.int16)
    same = ia == ib
    say(f"  outputs identical: {int(same.sum())} of {same.numel()}")
    assert bool(same.all())
    assert torch.equal(rings[0].view(torch.int16), rings[1].view(torch.int16))
    # the in-launch merge on its own against the storage-faithful oracle
    got = f64(outs[0])
    for l in range(L):
        for s in range(min(S, ORACLE_STREAMS)):
            qh, kh, vh = (f64(x)[:, l, s] for x in (qc, kc, vc))
            o = int(origins[s])
            if mode == "rebase":
                sim = stg.RebaseRing(HQ, HKV, D, W, dc, 1e6, origin=o,
                                     compensated=flags == "comp")
            else:
                sim = stg.CompactBuffer(HQ, HKV, D, W, cap, 1e6, origin=o)
            sf = np.stack([sim.step(qh[t % T], kh[t % T], vh[t % T])[1] for t in range(steps)])
            check_close(got[:, l, s], sf, 1e-3,
                        f"{name} l{l} s{s} vs storage-faithful", ulp_slack=True)


def test_encoder_chunks_merge_in_launch():
    """Encoder chunks with split key ranges: in-launch merge against the merge
    launch, bit for bit."""
    rkv = rkv_mod()
    dev = device()
    L, S, H, d, F, W, steps = 1, 2, 4, 64, 4, 60, 40
    cap = W + F
    origins = np.array([0, 17], np.int64)
    _, _, _, q, k, v = _pool(4200, (steps, L, S, F, H, d), (steps, L, S, F, H, d), dev)
    outs, rings = [], []
    for merge_flag in (0, rkv.RKV_F_MERGE_LAUNCH):
        cfg = rkv.make_cfg(S, L, num_q_heads=H, num_kv_heads=H, head_dim=d,
                           mode=rkv.RKV_MODE_ENC_CHUNK, new_rows=F, num_splits=3,
                           flags=merge_flag)
        cache = rkv.Cache(cfg, cap, W, cap, origins, device=dev)
        out = torch.full((steps, L, S, F, H, d), float("nan"), dtype=torch.bfloat16, device=dev)
        for t in range(steps):
            rkv.rkv_advance(cfg, cache.state, cache.plan)
            rkv.rkv_encoder_chunk_attn(cfg, cache.plan, cache.kv, q[t], k[t], v[t], out[t],
                                       cache.workspace)
        torch.cuda.synchronize()
        if not merge_flag:
            _counters_zero(rkv, cfg, cache)
        outs.append(out)
        rings.append(cache.buf)
    assert bool(torch.isfinite(outs[0].float()).all())
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    assert torch.equal(rings[0].view(torch.int16), rings[1].view(torch.int16))
