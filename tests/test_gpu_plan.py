"""rkv_advance against the oracle schedule: integer plan fields bit-exact for
every stream and step, float64 rotary tables equal to NumPy's cos/sin of
the same float64 angles within a few float64 ulps."""
import numpy as np
import pytest
import torch

from oracle import rope
from oracle import schedule as sch

from gpu_util import device, rkv_mod, say

pytestmark = pytest.mark.gpu

FIELDS = ("t", "pos", "pos_offset", "first_pos", "evict_pos", "slot", "n_valid",
          "rebase_delta", "compact_drop", "evict_slot", "window", "cap", "new_rows")


def _run(rkv, cfg, windows, caps, origins, steps, dc, F):
    dev = device()
    S = cfg.num_streams
    cfg.max_cap = int(np.max(caps))
    host = rkv.rkv_state_init_host(cfg, windows, caps, origins)
    state = torch.from_numpy(host.view(np.uint8).copy()).to(dev)
    plan = torch.zeros(S * rkv.PLAN_DTYPE.itemsize, dtype=torch.uint8, device=dev)
    got = []
    for _ in range(steps):
        rkv.rkv_advance(cfg, state, plan)
        got.append(plan.clone())
    torch.cuda.synchronize()
    got = [g.cpu().numpy().view(rkv.PLAN_DTYPE) for g in got]
    d = cfg.head_dim
    for s in range(S):
        st = sch.init_state(cfg.mode, int(windows[s]), int(caps[s]), int(origins[s]), dc, F)
        for i in range(steps):
            ref = sch.step(cfg.mode, st, dc, F).as_dict()
            row = got[i][s]
            for f in FIELDS:
                assert int(row[f]) == ref[f], (s, i, f, int(row[f]), ref[f])
            if i % 97 == 0 or ref["rebase_delta"]:
                pos = ref["pos"] + np.arange(F)
                ang = rope.angles(pos, d, cfg.rope_base)            # [F, d/2]
                np.testing.assert_allclose(row["rope_new"][:F, 0, :d // 2], np.cos(ang), atol=1e-14)
                np.testing.assert_allclose(row["rope_new"][:F, 1, :d // 2], np.sin(ang), atol=1e-14)
                dang = rope.angles(ref["rebase_delta"], d, cfg.rope_base)
                np.testing.assert_allclose(row["rope_delta"][0, :d // 2], np.cos(dang), atol=1e-14)
                np.testing.assert_allclose(row["rope_delta"][1, :d // 2], np.sin(dang), atol=1e-14)
    say(f"plan mode {cfg.mode}: {S} streams x {steps} steps bit-exact")


def test_plan_rebase_mixed_windows():
    rkv = rkv_mod()
    S = 6
    cfg = rkv.make_cfg(S, 1, rebase_chunk=25)
    windows = np.array([375, 250, 188, 375, 250, 188], np.int32)
    origins = np.array([0, 17, 4999, 25, 1, 600], np.int64)
    _run(rkv, cfg, windows, windows, origins, 500, 25, 1)


def test_plan_rebase_every_step():
    rkv = rkv_mod()
    cfg = rkv.make_cfg(2, 1, rebase_chunk=1, flags=rkv.RKV_F_COMPENSATED)
    _run(rkv, cfg, np.array([375, 7], np.int32), np.array([375, 7], np.int32),
         np.array([0, 3], np.int64), 420, 1, 1)


def test_plan_compaction():
    rkv = rkv_mod()
    cfg = rkv.make_cfg(3, 1, mode=rkv.RKV_MODE_COMPACT)
    windows = np.array([8, 64, 5], np.int32)
    caps = np.array([12, 80, 6], np.int32)
    _run(rkv, cfg, windows, caps, np.array([0, 9, 123456], np.int64), 300, 1, 1)


def test_plan_encoder_ring():
    rkv = rkv_mod()
    cfg = rkv.make_cfg(3, 1, num_q_heads=20, num_kv_heads=20, head_dim=64,
                       mode=rkv.RKV_MODE_ENC_CHUNK, new_rows=4)
    windows = np.array([750, 30, 30], np.int32)
    caps = np.array([754, 34, 40], np.int32)
    _run(rkv, cfg, windows, caps, np.array([0, 0, 8], np.int64), 260, 1, 4)


def test_device_state_init_equals_host_build():
    """rkv_state_init writes the same bytes as rkv_state_init_host, over more
    streams than one host chunk (mixed windows and start offsets)."""
    rkv = rkv_mod()
    dev = device()
    S = 300
    say(f"state init: S={S}")
    cfg = rkv.make_cfg(S, 2, rebase_chunk=25, max_cap=375)
    rng = np.random.default_rng(7)
    windows = rng.choice(np.array([375, 250, 188], np.int32), S)
    origins = rng.integers(0, 5000, S).astype(np.int64)
    state = torch.full((S * rkv.STATE_DTYPE.itemsize,), 0xAB, dtype=torch.uint8, device=dev)
    rkv.rkv_state_init(cfg, state, windows, windows, origins)
    got = state.cpu().numpy()
    ref = rkv.rkv_state_init_host(cfg, windows, windows, origins).view(np.uint8)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("mode", ["rebase", "compact", "encoder"])
def test_host_advance_equals_device_advance(mode):
    """rkv_state_advance_host(n) leaves the same state bytes as n rkv_advance
    launches (the bench starts its counter runs from such a state)."""
    rkv = rkv_mod()
    dev = device()
    if mode == "rebase":
        cfg = rkv.make_cfg(3, 1, rebase_chunk=25, max_cap=375)
        w = c = np.array([375, 250, 188], np.int32)
        steps = 437
    elif mode == "compact":
        cfg = rkv.make_cfg(3, 1, mode=rkv.RKV_MODE_COMPACT, max_cap=80)
        w, c = np.array([64, 8, 5], np.int32), np.array([80, 12, 6], np.int32)
        steps = 301
    else:
        cfg = rkv.make_cfg(2, 1, num_q_heads=20, num_kv_heads=20, head_dim=64,
                           mode=rkv.RKV_MODE_ENC_CHUNK, new_rows=4, max_cap=754)
        w, c = np.array([750, 30], np.int32), np.array([754, 34], np.int32)
        steps = 200
    o = np.arange(cfg.num_streams, dtype=np.int64) * 11
    say(f"host advance vs device: mode={mode} steps={steps}")
    host = rkv.rkv_state_init_host(cfg, w, c, o)
    state = torch.from_numpy(host.view(np.uint8).copy()).to(dev)
    plan = torch.zeros(cfg.num_streams * rkv.PLAN_DTYPE.itemsize, dtype=torch.uint8, device=dev)
    for _ in range(steps):
        rkv.rkv_advance(cfg, state, plan)
    torch.cuda.synchronize()
    rkv.rkv_state_advance_host(cfg, host, steps)
    assert np.array_equal(state.cpu().numpy(), host.view(np.uint8))
