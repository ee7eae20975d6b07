"""Continuous-mode decoder restart on the GPU (voxtral.c explainer, section
四: a hard decoder reset, no context kept): rkv_reset_streams against the
host-side initial states, a pipelined loop restarted mid-run against the
rkv_advance loop restarted at the same step (bit for bit), and end-to-end
attention after a restart against the float64 oracle of a fresh stream."""
import numpy as np
import pytest
import torch

from oracle import attention as att
from rolling_window_kv_amd import synth

from gpu_util import check_close, device, f64, rkv_mod, say

pytestmark = pytest.mark.gpu

HEADER = ("t", "pos", "pos_offset", "first_pos", "evict_pos", "slot", "n_valid",
          "rebase_delta", "compact_drop", "evict_slot", "window", "cap", "new_rows")


def _state_bytes(cache):
    return cache.state_host().view(np.uint8).reshape(len(cache.state_host()), -1)


def test_reset_writes_initial_states_and_keeps_the_others():
    rkv = rkv_mod()
    dev = device()
    S, W, dc = 70, 40, 5                  # 70 streams: the list spans two launches
    say(f"reset states: S={S} W={W} dc={dc}")
    cfg = rkv.make_cfg(S, 1, rebase_chunk=dc)
    origins = np.arange(S, dtype=np.int64) * 7
    cache = rkv.Cache(cfg, W, W, W, origins, device=dev)
    for _ in range(53):
        rkv.rkv_advance(cfg, cache.state, cache.plan)
    torch.cuda.synchronize()
    before = cache.state_host().copy()
    streams = list(range(0, 66)) + [3]    # 66 distinct, then stream 3 again
    new_origin = [1000 + 3 * s for s in range(66)] + [5]
    rkv.rkv_reset_streams(cfg, cache.state, None, streams, new_origin)
    torch.cuda.synchronize()
    after = cache.state_host()
    final = {s: o for s, o in zip(streams, new_origin)}      # the later origin wins
    win = np.full(S, W, np.int32)
    org = np.array([final.get(s, 0) for s in range(S)], np.int64)
    init = rkv.rkv_state_init_host(cfg, win, win, org)
    for s in range(S):
        want = init[s] if s in final else before[s]
        assert after[s].tobytes() == want.tobytes(), f"stream {s}"


@pytest.mark.parametrize("mode,S,L,W,cap,dc", [(0, 5, 2, 40, 40, 5), (1, 3, 2, 24, 30, 1)])
def test_pipelined_restart_matches_advance_loop(mode, S, L, W, cap, dc):
    """Loop a: rkv_advance + rkv_decode_step, restart before rkv_advance.
    Loop b: pipelined, restart with the already written next plan.  Outputs,
    rings, states and plans agree bit for bit before and after the restart."""
    rkv = rkv_mod()
    dev = device()
    say(f"pipelined restart: mode={mode} S={S} L={L} W={W} cap={cap} dc={dc}")
    cfg = rkv.make_cfg(S, L, mode=mode, rebase_chunk=dc)
    origins = np.arange(S, dtype=np.int64) * 3
    a = rkv.Cache(cfg, cap, W, cap, origins, device=dev)
    b = rkv.Cache(cfg, cap, W, cap, origins, device=dev)
    gen = torch.Generator().manual_seed(31)
    P = 5
    q = torch.randn((P, L, S, 16, 128), generator=gen).to(torch.bfloat16).to(dev)
    k = torch.randn((P, L, S, 2, 128), generator=gen).to(torch.bfloat16).to(dev)
    v = torch.randn((P, L, S, 2, 128), generator=gen).to(torch.bfloat16).to(dev)
    oa = torch.empty(q.shape[1:], dtype=torch.bfloat16, device=dev)
    ob = torch.empty_like(oa)
    plans = [b.plan, b.plan_next]
    rkv.rkv_advance(cfg, b.state, plans[0])
    restart_at, streams, new_origin = 67, [0, S - 1], [500, 0]
    for i in range(2 * restart_at):
        j = i % P
        if i == restart_at:
            rkv.rkv_reset_streams(cfg, a.state, None, streams, new_origin)
            rkv.rkv_reset_streams(cfg, b.state, plans[i % 2], streams, new_origin)
        rkv.rkv_advance(cfg, a.state, a.plan)
        cur, nxt = plans[i % 2], plans[(i + 1) % 2]
        if i == restart_at:
            torch.cuda.synchronize()
            pa = a.plan_host()
            pb = cur.cpu().numpy().view(rkv.PLAN_DTYPE)
            for f in HEADER:
                assert np.array_equal(pa[f], pb[f]), f
            assert np.array_equal(_state_bytes(a), _state_bytes(b))
            assert np.all(pa["n_valid"][streams] == 1)
        if mode == 1:
            rkv.rkv_compact(cfg, a.plan, a.kv)
            rkv.rkv_compact(cfg, cur, b.kv)
        rkv.rkv_decode_step(cfg, a.plan, a.kv, q[j], k[j], v[j], oa, a.workspace)
        rkv.rkv_decode_step_pipelined(cfg, b.state, cur, nxt, b.kv, q[j], k[j], v[j], ob,
                                      b.workspace)
        assert torch.equal(oa, ob), f"output differs at step {i}"
    torch.cuda.synchronize()
    assert torch.equal(a.buf, b.buf)


def test_restarted_stream_attends_only_to_its_new_context():
    """Three streams, 2 layers, W = 40, re-base chunk 5: after 70 steps stream
    1 restarts at position 0 and stream 2 at 1000; 60 more steps.  Stream 0
    matches the oracle over its whole history, streams 1 and 2 the oracle of a
    fresh stream fed only the inputs after the restart (a stale row in the
    window would be far outside the 2e-2 gate)."""
    rkv = rkv_mod()
    dev = device()
    S, L, W, dc, T1, T2 = 3, 2, 40, 5, 70, 60
    say(f"restart end-to-end: S={S} L={L} W={W} dc={dc} steps {T1}+{T2}")
    q, k, v = synth.decoder_pool(2024, L, S, T1 + T2, 16, 2, 128)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    cfg = rkv.make_cfg(S, L, rebase_chunk=dc)
    cache = rkv.Cache(cfg, W, W, W, 0, device=dev)
    out = torch.zeros((T1 + T2,) + tuple(q.shape[1:]), dtype=torch.bfloat16, device=dev)
    for t in range(T1 + T2):
        if t == T1:
            rkv.rkv_reset_streams(cfg, cache.state, None, [1, 2], [0, 1000])
        rkv.rkv_advance(cfg, cache.state, cache.plan)
        rkv.rkv_decode_step(cfg, cache.plan, cache.kv, qd[t], kd[t], vd[t], out[t],
                            cache.workspace)
    torch.cuda.synchronize()
    got = f64(out)
    qh, kh, vh = f64(q), f64(k), f64(v)
    for l in range(L):
        whole = att.window_decode(qh[:, l, 0], kh[:, l, 0], vh[:, l, 0], W, 1e6)
        check_close(got[:, l, 0], np.stack([whole[t] for t in range(T1 + T2)]), 2e-2,
                    f"layer {l} stream 0 (kept)")
        for s, origin in ((1, 0), (2, 1000)):
            fresh = att.window_decode(qh[T1:, l, s], kh[T1:, l, s], vh[T1:, l, s], W, 1e6,
                                      origin=origin)
            check_close(got[T1:, l, s], np.stack([fresh[t] for t in range(T2)]), 2e-2,
                        f"layer {l} stream {s} (restarted at {origin})")
