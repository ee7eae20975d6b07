"""rkv_decode_step_pipelined, and rkv_update_step + rkv_decode_attn_pipelined,
against rkv_advance + rkv_decode_step: the same outputs, rings, states and
plans, bit for bit, when the caller alternates two plan buffers (re-base
steps, compaction steps, a split key range and a stream count that leaves
part of the last plan block idle)."""
import numpy as np
import pytest
import torch

from gpu_util import device, rkv_mod, say

pytestmark = pytest.mark.gpu

HEADER = ("t", "pos", "pos_offset", "first_pos", "evict_pos", "slot", "n_valid",
          "rebase_delta", "compact_drop", "evict_slot", "window", "cap", "new_rows")


def _pair(rkv, cfg, slots, W, cap, origins, dev):
    return [rkv.Cache(cfg, slots, W, cap, origins, device=dev) for _ in range(2)]


@pytest.mark.parametrize("path", ["fused", "update"])
@pytest.mark.parametrize("mode,S,L,W,cap,dc,steps", [
    (0, 5, 2, 40, 40, 5, 130),        # re-base every 5 positions once the window is full
    (1, 3, 2, 24, 30, 1, 90),         # compaction every 7 steps after the first fill
    (0, 1, 1, 375, 375, 25, 420),     # one item, the key range split 6 ways
])
def test_pipelined_step_matches_advance_then_step(mode, S, L, W, cap, dc, steps, path):
    rkv = rkv_mod()
    dev = device()
    say(f"pipelined ({path}): mode={mode} S={S} L={L} W={W} cap={cap} dc={dc} steps={steps}")
    cfg = rkv.make_cfg(S, L, mode=mode, rebase_chunk=dc, num_splits=6 if S == 1 else 0)
    origins = np.arange(S, dtype=np.int64) * 3
    a, b = _pair(rkv, cfg, cap, W, cap, origins, dev)
    gen = torch.Generator().manual_seed(21)
    P = 7
    q = torch.randn((P, L, S, 16, 128), generator=gen).to(torch.bfloat16).to(dev)
    k = torch.randn((P, L, S, 2, 128), generator=gen).to(torch.bfloat16).to(dev)
    v = torch.randn((P, L, S, 2, 128), generator=gen).to(torch.bfloat16).to(dev)
    oa = torch.empty(q.shape[1:], dtype=torch.bfloat16, device=dev)
    ob = torch.empty_like(oa)
    plans = [b.plan, b.plan_next]
    rkv.rkv_advance(cfg, b.state, plans[0])
    rebases = drops = 0
    for i in range(steps):
        j = i % P
        rkv.rkv_advance(cfg, a.state, a.plan)
        cur, nxt = plans[i % 2], plans[(i + 1) % 2]
        if mode == 1:
            rkv.rkv_compact(cfg, a.plan, a.kv)
            rkv.rkv_compact(cfg, cur, b.kv)
        rkv.rkv_decode_step(cfg, a.plan, a.kv, q[j], k[j], v[j], oa, a.workspace)
        if path == "update":
            rkv.rkv_update_step(cfg, cur, b.kv, k[j], v[j])
            rkv.rkv_decode_attn_pipelined(cfg, b.state, cur, nxt, b.kv, q[j], ob, b.workspace)
        else:
            rkv.rkv_decode_step_pipelined(cfg, b.state, cur, nxt, b.kv, q[j], k[j], v[j], ob,
                                          b.workspace)
        pa = a.plan_host()
        rebases += int((pa["rebase_delta"] != 0).sum())
        drops += int((pa["compact_drop"] != 0).sum())
        assert torch.equal(oa, ob), f"output differs at step {i}"
    torch.cuda.synchronize()
    assert torch.equal(a.buf, b.buf)
    # the pipelined run has already planned the next step: do the same on a
    rkv.rkv_advance(cfg, a.state, a.plan)
    torch.cuda.synchronize()
    assert np.array_equal(a.state_host().view(np.uint8), b.state_host().view(np.uint8))
    pa = a.plan_host()
    pb = plans[steps % 2].cpu().numpy().view(rkv.PLAN_DTYPE)
    for f in HEADER:
        assert np.array_equal(pa[f], pb[f]), f
    half = cfg.head_dim // 2
    assert np.array_equal(pa["rope_new"][:, 0, :, :half], pb["rope_new"][:, 0, :, :half])
    assert np.array_equal(pa["rope_delta"][:, :, :half], pb["rope_delta"][:, :, :half])
    say(f"  re-base plans seen {rebases}, compaction plans seen {drops}")
    if mode == 0 and dc > 1:
        assert rebases > 0
    if mode == 1:
        assert drops > 0
