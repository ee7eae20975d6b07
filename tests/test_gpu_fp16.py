"""The fp16 cache variant (RKV_F_KV_FP16; voxtral.c explainer, section 七,
fp16 KV cache) against the float64 oracle with binary16 storage rounding:
per call, appended and re-based K within one binary16 ulp and V exactly the
binary16 rounding of the bfloat16 input; end to end, attention within 2e-2 of
the exact oracle and within 1e-3 + 1 bf16 ulp of the storage-faithful fp16
simulation (re-base chunks of 25 and of 1, and compaction; re-basing by 1
without the compensating residual against the simulation only); and the fused,
separate and pipelined paths writing the same bits."""
import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import fp16 as of
from oracle import storage as stg
from rolling_window_kv_amd import synth

from gpu_util import check_close, device, f64, rkv_mod, run_decoder, say

pytestmark = pytest.mark.gpu

HQ, HKV, D = 16, 2, 128


def _ulp(got, want, label, max_ulp=1):
    d = of.ulp_distance(got, want)
    say(f"{label}: max ulp {int(d.max())}, exact {float((d == 0).mean()):.6f}")
    assert d.max() <= max_ulp


@pytest.mark.parametrize("dc,comp", [(1, False), (1, True), (5, False)])
def test_fp16_rebase_call_within_one_ulp(dc, comp):
    rkv = rkv_mod()
    dev = device()
    L, S, W = 2, 3, 45
    flags = rkv.RKV_F_KV_FP16 | (rkv.RKV_F_COMPENSATED if comp else 0)
    cfg = rkv.make_cfg(S, L, rebase_chunk=dc, flags=flags)
    cache = rkv.Cache(cfg, W, W, W, 0, device=dev)
    for _ in range(100000):
        rkv.rkv_advance(cfg, cache.state, cache.plan)
        p = cache.plan_host()
        if p["rebase_delta"][0] > 0:
            break
    gen = torch.Generator().manual_seed(41)
    x = torch.randn(cache.k.shape, generator=gen).to(torch.float16)
    cache.k.copy_(x)
    if comp:
        xlo = (torch.randn(cache.k.shape, generator=gen) * 2.0 ** -13).to(torch.float16)
        cache.k_lo.copy_(xlo)
    rkv.rkv_roll_rebase(cfg, cache.plan, cache.kv)
    torch.cuda.synchronize()
    got = f64(cache.k)
    x64 = f64(x)
    lo64 = f64(xlo) if comp else np.zeros_like(x64)
    delta = int(p["rebase_delta"][0])
    rows = [r for r in range(int(p["n_valid"][0])) if r != int(p["slot"][0])]
    want_hi, want_lo = stg.rebase_k(x64[:, :, :, rows], lo64[:, :, :, rows], delta,
                                    cfg.rope_base, comp, rounder=of.round_f16)
    _ulp(got[:, :, :, rows], want_hi, f"fp16 rebase dc={dc} comp={comp}")
    untouched = [r for r in range(W) if r not in rows]
    assert np.array_equal(got[:, :, :, untouched], x64[:, :, :, untouched])
    if comp:
        # hi + lo carries ~22 significant bits, except that lo cannot go below
        # binary16's subnormal quantum 2^-24: an absolute floor of two quanta
        glo = f64(cache.k_lo)[:, :, :, rows]
        y = want_hi + want_lo
        err = np.abs(got[:, :, :, rows] + glo - y)
        assert np.all(err <= 2.0 ** -20 * np.abs(y) + 2.0 ** -23), float(err.max())


@pytest.mark.parametrize("mode,comp", [(0, False), (0, True), (1, False)])
def test_fp16_append_call(mode, comp):
    rkv = rkv_mod()
    dev = device()
    L, S, W = 2, 3, 20
    cap = W if mode == 0 else W + 6
    flags = rkv.RKV_F_KV_FP16 | (rkv.RKV_F_COMPENSATED if comp else 0)
    cfg = rkv.make_cfg(S, L, mode=mode, rebase_chunk=1, flags=flags)
    origins = np.array([0, 5, 1000003], np.int64)
    cache = rkv.Cache(cfg, cap, W, cap, origins, device=dev)
    gen = torch.Generator().manual_seed(42)
    for step in range(2 * cap):
        rkv.rkv_advance(cfg, cache.state, cache.plan)
        if mode == 1:
            rkv.rkv_compact(cfg, cache.plan, cache.kv)
        kn = torch.randn((L, S, HKV, D), generator=gen).to(torch.bfloat16)
        vn = torch.randn((L, S, HKV, D), generator=gen).to(torch.bfloat16)
        vn[0, 0, 0, :4] = torch.tensor([1e-6, -3e-7, 7e4, 1e-9]).to(torch.bfloat16)
        rkv.rkv_append(cfg, cache.plan, cache.kv, kn.to(dev), vn.to(dev))
        torch.cuda.synchronize()
        if step % 5:
            continue
        p = cache.plan_host()
        gk, gv = f64(cache.k), f64(cache.v)
        for s in range(S):
            slot, pos = int(p["slot"][s]), int(p["pos"][s])
            hi, lo = stg.append_k(f64(kn)[:, s], pos, cfg.rope_base, comp, rounder=of.round_f16)
            _ulp(gk[:, s, :, slot], hi, f"fp16 append mode {mode} step {step} s{s}")
            want_v = of.round_f16(f64(vn)[:, s])
            assert np.array_equal(gv[:, s, :, slot], want_v, equal_nan=True)
            if comp:
                glo = f64(cache.k_lo)[:, s, :, slot]
                assert np.max(np.abs(gk[:, s, :, slot] + glo - (hi + lo))) <= np.max(
                    of.f16_ulp(lo))


@pytest.mark.parametrize("W,dc,T,comp,exact_gate,sf_gate", [
    (120, 25, 300, False, 2e-2, 1e-3),
    (375, 1, 500, True, 2e-2, 1e-3),
    # plain re-rounding every step, no residual: with 11 significant bits
    # fewer rotary pairs stall than in bfloat16, but the error against the
    # exact oracle still reaches ~3e-2 over 1000 steps (measured; ~1e-2 over
    # 500), so the compensated residual stays necessary for the 2e-2 gate and
    # this case is checked against the storage simulation only (which stalls
    # the same way); GPU and oracle re-rounding trajectories may part by an
    # ulp at ties, hence 2e-3
    (375, 1, 1000, False, None, 2e-3),
])
def test_fp16_decode_matches_oracles(W, dc, T, comp, exact_gate, sf_gate):
    rkv = rkv_mod()
    dev = device()
    S, L = 2, 2
    say(f"fp16 decode: W={W} dc={dc} T={T} comp={comp}")
    q, k, v = synth.decoder_pool(4242, L, S, T, HQ, HKV, D)
    flags = rkv.RKV_F_KV_FP16 | (rkv.RKV_F_COMPENSATED if comp else 0)
    cfg = rkv.make_cfg(S, L, rebase_chunk=dc, flags=flags)
    _, out, _ = run_decoder(rkv, cfg, W, W, W, 0, q.to(dev), k.to(dev), v.to(dev), True)
    got = f64(out)
    qh, kh, vh = f64(q), f64(k), f64(v)
    for l in range(L):
        for s in range(S):
            exact = att.window_decode(qh[:, l, s], kh[:, l, s], vh[:, l, s], W, 1e6)
            ex = np.stack([exact[t] for t in range(T)])
            if exact_gate is None:
                say(f"l{l} s{s} vs exact (no gate): max|err| {np.abs(got[:, l, s] - ex).max():.3e}")
            else:
                check_close(got[:, l, s], ex, exact_gate, f"l{l} s{s} vs exact")
            ring = stg.RebaseRing(HQ, HKV, D, W, dc, 1e6, compensated=comp,
                                  rounder=of.round_f16)
            sf = np.stack([ring.step(qh[t, l, s], kh[t, l, s], vh[t, l, s])[1] for t in range(T)])
            check_close(got[:, l, s], sf, sf_gate, f"l{l} s{s} vs fp16 storage", ulp_slack=True)


def test_fp16_compaction_matches_oracle():
    rkv = rkv_mod()
    dev = device()
    S, L, W, cap, T = 2, 1, 48, 60, 160
    q, k, v = synth.decoder_pool(4343, L, S, T, HQ, HKV, D)
    cfg = rkv.make_cfg(S, L, mode=rkv.RKV_MODE_COMPACT, flags=rkv.RKV_F_KV_FP16)
    _, out, _ = run_decoder(rkv, cfg, cap, W, cap, 0, q.to(dev), k.to(dev), v.to(dev), True)
    got = f64(out)
    qh, kh, vh = f64(q), f64(k), f64(v)
    for s in range(S):
        buf = stg.CompactBuffer(HQ, HKV, D, W, cap, 1e6, rounder=of.round_f16)
        sf = np.stack([buf.step(qh[t, 0, s], kh[t, 0, s], vh[t, 0, s])[1] for t in range(T)])
        check_close(got[:, 0, s], sf, 1e-3, f"compaction s{s} vs fp16 storage", ulp_slack=True)


def test_fp16_fused_separate_and_pipelined_write_the_same_bits():
    rkv = rkv_mod()
    dev = device()
    S, L, W, dc, T = 3, 2, 40, 5, 120
    q, k, v = (x.to(dev) for x in synth.decoder_pool(4444, L, S, 7, HQ, HKV, D))
    cfg = rkv.make_cfg(S, L, rebase_chunk=dc, flags=rkv.RKV_F_KV_FP16)
    a, oa, _ = run_decoder(rkv, cfg, W, W, W, 0, q, k, v, True, steps=T)
    b, ob, _ = run_decoder(rkv, cfg, W, W, W, 0, q, k, v, False, steps=T)
    assert torch.equal(oa, ob)
    assert torch.equal(a.buf, b.buf)
    c = rkv.Cache(cfg, W, W, W, 0, device=dev)
    oc = torch.empty_like(oa)
    plans = [c.plan, c.plan_next]
    rkv.rkv_advance(cfg, c.state, plans[0])
    for t in range(T):
        rkv.rkv_decode_step_pipelined(cfg, c.state, plans[t % 2], plans[(t + 1) % 2], c.kv,
                                      q[t % 7], k[t % 7], v[t % 7], oc[t], c.workspace)
    torch.cuda.synchronize()
    assert torch.equal(oa, oc)
    assert torch.equal(a.buf, c.buf)
