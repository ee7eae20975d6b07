"""Per-call gates of the cache updates, from identical input:
append (rne(R(p) k)) and re-base (rne(R(-D) x)) within one bfloat16 ulp of
the float64 oracle, V and compaction moves bit-exact, untouched rows
unchanged, and the fused decode step writing the same bits as
rkv_roll_rebase + rkv_append."""
import numpy as np
import pytest
import torch

from oracle import bf16 as ob
from oracle import storage as stg

from gpu_util import device, f64, rkv_mod, say

pytestmark = pytest.mark.gpu


def _rand_bf16(shape, gen, scale=1.0):
    return (torch.randn(shape, generator=gen) * scale).to(torch.bfloat16)


def _advance_until(rkv, cfg, cache, pred, limit=100000):
    for _ in range(limit):
        rkv.rkv_advance(cfg, cache.state, cache.plan)
        p = cache.plan_host()
        if pred(p):
            return p
    raise AssertionError("condition not reached")


def _assert_ulp(got, want, label, max_ulp=1):
    d = ob.ulp_distance(got, want)
    frac = float((d == 0).mean())
    say(f"{label}: max ulp {int(d.max())}, exact {frac:.6f}")
    assert d.max() <= max_ulp
    return frac


@pytest.mark.parametrize("dc,comp,d", [(1, False, 128), (1, True, 128), (5, False, 128),
                                       (3, True, 64)])
def test_rebase_call_matches_oracle(dc, comp, d):
    rkv = rkv_mod()
    dev = device()
    L, S, H, W = 2, 3, 2, 45
    flags = rkv.RKV_F_COMPENSATED if comp else 0
    cfg = rkv.make_cfg(S, L, num_q_heads=8 * H, num_kv_heads=H, head_dim=d, rebase_chunk=dc,
                       flags=flags)
    cache = rkv.Cache(cfg, W, W, W, 0, device=dev)
    p = _advance_until(rkv, cfg, cache, lambda p: p["rebase_delta"][0] > 0)
    gen = torch.Generator().manual_seed(11)
    x = _rand_bf16(cache.k.shape, gen)
    cache.k.copy_(x)
    if comp:
        xlo = _rand_bf16(cache.k.shape, gen, 2.0 ** -10)
        cache.k_lo.copy_(xlo)
    rkv.rkv_roll_rebase(cfg, cache.plan, cache.kv)
    torch.cuda.synchronize()
    got = f64(cache.k)
    x64 = f64(x)
    lo64 = f64(xlo) if comp else np.zeros_like(x64)
    delta = int(p["rebase_delta"][0])
    n_valid, slot = int(p["n_valid"][0]), int(p["slot"][0])
    rows = [r for r in range(n_valid) if r != slot]
    want_hi, want_lo = stg.rebase_k(x64[:, :, :, rows], lo64[:, :, :, rows], delta,
                                    cfg.rope_base, comp)
    _assert_ulp(got[:, :, :, rows], want_hi, f"rebase dc={dc} comp={comp} d={d} hi")
    untouched = [r for r in range(W) if r not in rows]
    assert np.array_equal(got[:, :, :, untouched], x64[:, :, :, untouched])
    if comp:
        glo = f64(cache.k_lo)[:, :, :, rows]
        y = want_hi + want_lo
        assert np.max(np.abs(got[:, :, :, rows] + glo - y) / (np.abs(y) + 1e-30)) < 2.0 ** -15


@pytest.mark.parametrize("mode,d,comp", [(0, 128, False), (0, 128, True), (1, 128, False),
                                         (2, 64, False)])
def test_append_call_matches_oracle(mode, d, comp):
    rkv = rkv_mod()
    dev = device()
    L, S = 2, 3
    if mode == 2:
        H, F, W, cap = 4, 4, 10, 14
        cfg = rkv.make_cfg(S, L, num_q_heads=H, num_kv_heads=H, head_dim=d, mode=mode, new_rows=F)
        in_shape = (L, S, F, H, d)
    else:
        H, F, W = 2, 1, 20
        cap = W if mode == 0 else W + 6
        cfg = rkv.make_cfg(S, L, num_kv_heads=H, head_dim=d, mode=mode, rebase_chunk=1,
                           flags=rkv.RKV_F_COMPENSATED if comp else 0)
        in_shape = (L, S, H, d)
    origins = np.array([0, 5, 1000003], np.int64)
    cache = rkv.Cache(cfg, cap, W, cap, origins, device=dev)
    gen = torch.Generator().manual_seed(12)
    for step in range(3 * cap):
        rkv.rkv_advance(cfg, cache.state, cache.plan)
        if mode == 1:
            rkv.rkv_compact(cfg, cache.plan, cache.kv)
        kn = _rand_bf16(in_shape, gen).to(dev)
        vn = _rand_bf16(in_shape, gen).to(dev)
        before_k = cache.k.clone()
        rkv.rkv_append(cfg, cache.plan, cache.kv, kn, vn)
        torch.cuda.synchronize()
        if step % 7 and step < 3 * cap - 1:
            continue
        p = cache.plan_host()
        gk, bk, gv = f64(cache.k), f64(before_k), f64(cache.v)
        kn64, vn64 = f64(kn), f64(vn)
        touched = np.zeros(gk.shape[:4], bool)
        for s in range(S):
            for j in range(F):
                slot = (int(p["slot"][s]) + j) % int(p["cap"][s])
                pos = int(p["pos"][s]) + j
                src_k = kn64[:, s, j] if mode == 2 else kn64[:, s]
                src_v = vn64[:, s, j] if mode == 2 else vn64[:, s]
                hi, lo = stg.append_k(src_k, pos, cfg.rope_base, comp)
                _assert_ulp(gk[:, s, :, slot], hi, f"append mode {mode} step {step} s{s} j{j}")
                assert np.array_equal(gv[:, s, :, slot], src_v)
                touched[:, s, :, slot] = True
                if comp:
                    glo = f64(cache.k_lo)[:, s, :, slot]
                    same = ob.ulp_distance(gk[:, s, :, slot], hi) == 0
                    assert ob.ulp_distance(glo[same], lo[same]).max() <= 1
        assert np.array_equal(gk[~touched], bk[~touched])


@pytest.mark.parametrize("W,cap,d", [(64, 80, 128), (100, 250, 128), (40, 47, 64),
                                     (30, 31, 128), (8192, 9216, 128)])
def test_compaction_move_is_exact(W, cap, d):
    rkv = rkv_mod()
    dev = device()
    L, S, H = (1, 2, 2) if W > 1000 else (2, 3, 2)
    cfg = rkv.make_cfg(S, L, num_kv_heads=H, head_dim=d, mode=rkv.RKV_MODE_COMPACT)
    cache = rkv.Cache(cfg, cap, W, cap, 0, device=dev)
    p = _advance_until(rkv, cfg, cache, lambda p: p["compact_drop"][0] > 0)
    drop = int(p["compact_drop"][0])
    assert drop == cap - W
    gen = torch.Generator().manual_seed(13)
    xk = _rand_bf16(cache.k.shape, gen).to(dev)
    xv = _rand_bf16(cache.v.shape, gen).to(dev)
    cache.k.copy_(xk)
    cache.v.copy_(xv)
    rkv.rkv_compact(cfg, cache.plan, cache.kv)
    torch.cuda.synchronize()
    assert torch.equal(cache.k[:, :, :, :W], xk[:, :, :, drop:drop + W])
    assert torch.equal(cache.v[:, :, :, :W], xv[:, :, :, drop:drop + W])
    assert torch.equal(cache.k[:, :, :, W:], xk[:, :, :, W:])
    assert torch.equal(cache.v[:, :, :, W:], xv[:, :, :, W:])
    say(f"compaction W={W} cap={cap} d={d}: moved {W} rows exactly (drop {drop})")


@pytest.mark.parametrize("dc,comp", [(1, True), (4, False)])
def test_fused_step_writes_same_bits_as_separate_calls(dc, comp):
    rkv = rkv_mod()
    dev = device()
    L, S, H, W, d = 2, 3, 2, 50, 128
    flags = rkv.RKV_F_COMPENSATED if comp else 0
    cfg = rkv.make_cfg(S, L, num_kv_heads=H, head_dim=d, rebase_chunk=dc, flags=flags)
    origins = np.array([0, 3, 77], np.int64)
    a = rkv.Cache(cfg, W, W, W, origins, device=dev)
    b = rkv.Cache(cfg, W, W, W, origins, device=dev)
    gen = torch.Generator().manual_seed(14)
    qs = [_rand_bf16((L, S, 8 * H, d), gen).to(dev) for _ in range(4)]
    ks = [_rand_bf16((L, S, H, d), gen).to(dev) for _ in range(4)]
    vs = [_rand_bf16((L, S, H, d), gen).to(dev) for _ in range(4)]
    oa = torch.zeros((L, S, 8 * H, d), dtype=torch.bfloat16, device=dev)
    ob_ = torch.zeros_like(oa)
    for step in range(3 * W):
        i = step % 4
        for c in (a, b):
            rkv.rkv_advance(cfg, c.state, c.plan)
        rkv.rkv_roll_rebase(cfg, a.plan, a.kv)
        rkv.rkv_append(cfg, a.plan, a.kv, ks[i], vs[i])
        rkv.rkv_decode_attn(cfg, a.plan, a.kv, qs[i], oa, a.workspace)
        rkv.rkv_decode_step(cfg, b.plan, b.kv, qs[i], ks[i], vs[i], ob_, b.workspace)
        if step % 10 == 9:
            torch.cuda.synchronize()
            assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
            if comp:
                assert torch.equal(a.k_lo, b.k_lo)
            assert torch.equal(oa, ob_)
    say(f"fused == separate, dc={dc} comp={comp}: rings and outputs bit-identical")


@pytest.mark.parametrize("case", ["rebase_dc1_comp", "rebase_dc4", "rebase_fp16_comp",
                                  "encoder", "compact", "many_streams"])
def test_update_step_writes_same_bits_as_rebase_then_append(case):
    """rkv_update_step (one launch) against rkv_roll_rebase + rkv_append (and
    rkv_compact first in compaction mode): rings bit-identical after every
    step, with staggered stream origins so that some streams re-base in most
    steps; 8,300 streams take the moving-stream list through two passes."""
    rkv = rkv_mod()
    dev = device()
    gen = torch.Generator().manual_seed(15)
    L, S, H, d, W, cap, F, steps = 2, 5, 2, 128, 40, 40, 1, 90
    kw = dict(num_kv_heads=H, head_dim=d)
    origins = np.array([0, 3, 7, 11, 30], np.int64)
    if case == "rebase_dc1_comp":
        cfg = rkv.make_cfg(S, L, rebase_chunk=1, flags=rkv.RKV_F_COMPENSATED, **kw)
    elif case == "rebase_dc4":
        cfg = rkv.make_cfg(S, L, rebase_chunk=4, **kw)
    elif case == "rebase_fp16_comp":
        cfg = rkv.make_cfg(S, L, rebase_chunk=3,
                           flags=rkv.RKV_F_COMPENSATED | rkv.RKV_F_KV_FP16, **kw)
    elif case == "encoder":
        H, d, F = 4, 64, 4
        cfg = rkv.make_cfg(S, L, num_q_heads=H, num_kv_heads=H, head_dim=d,
                           mode=rkv.RKV_MODE_ENC_CHUNK, new_rows=F)
        cap = W + F
        origins = 0
    elif case == "compact":
        cap = 52
        cfg = rkv.make_cfg(S, L, mode=rkv.RKV_MODE_COMPACT, **kw)
    else:
        L, S, H, d, W, cap, steps = 1, 8300, 1, 64, 6, 6, 14
        cfg = rkv.make_cfg(S, L, num_q_heads=1, num_kv_heads=1, head_dim=d, rebase_chunk=2)
        origins = np.arange(S, dtype=np.int64) % 7
    a = rkv.Cache(cfg, cap, W, cap, origins, device=dev)
    b = rkv.Cache(cfg, cap, W, cap, origins, device=dev)
    shape = (L, S, F, H, d) if F > 1 else (L, S, H, d)
    ks = [_rand_bf16(shape, gen).to(dev) for _ in range(3)]
    vs = [_rand_bf16(shape, gen).to(dev) for _ in range(3)]
    moved = 0
    for step in range(steps):
        i = step % 3
        for c in (a, b):
            rkv.rkv_advance(cfg, c.state, c.plan)
            if case == "compact":
                rkv.rkv_compact(cfg, c.plan, c.kv)
        if step % 7 == 0:
            moved += int((a.plan_host()["rebase_delta"] != 0).sum())
        if cfg.mode == rkv.RKV_MODE_REBASE:
            rkv.rkv_roll_rebase(cfg, a.plan, a.kv)
        rkv.rkv_append(cfg, a.plan, a.kv, ks[i], vs[i])
        rkv.rkv_update_step(cfg, b.plan, b.kv, ks[i], vs[i])
        if step % 5 == 4 or step == steps - 1:
            torch.cuda.synchronize()
            assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v), step
            if a.k_lo is not None:
                assert torch.equal(a.k_lo, b.k_lo), step
    if cfg.mode == rkv.RKV_MODE_REBASE:
        assert moved > 0
    say(f"update step == re-base + append ({case}): rings bit-identical over {steps} steps")
