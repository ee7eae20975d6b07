"""Delay conditioning on the GPU (rkv_tcond_prepare, rkv_tcond_modulate)
against oracle.tcond: the modulation vectors of the eight post-trained
(clock, delay) settings, the in-place modulation of bfloat16 and float32
attention outputs with streams on different settings or none, and the
modulation of a full 36-layer x 64-stream decode step's output."""
import numpy as np
import pytest
import torch

from oracle import tcond
from oracle.bf16 import bf16_ulp
from rolling_window_kv_amd import synth

from gpu_util import device, f64, rkv_mod, say

pytestmark = pytest.mark.gpu

# the model card's post-trained (clock, delay) settings
SETTINGS = [(80, 240), (80, 320), (80, 480), (80, 560), (120, 240), (120, 480), (160, 320),
            (160, 480)]


def _prepare(rkv, L, hidden, dim, seed):
    dev = device()
    conds = [tcond.delay_tokens(dl, ck) for ck, dl in SETTINGS]
    n = [c[0] for c in conds]
    fl = [c[1] for c in conds]
    table, A = synth.tcond_weights(seed, L, hidden, dim)
    tc = rkv.make_tcond_cfg(L, hidden, dim=dim, num_conds=len(conds), max_frame_len=8)
    mod = torch.empty((L, len(conds), 2, hidden), dtype=torch.float32, device=dev)
    rkv.rkv_tcond_prepare(tc, n, fl, table.to(dev), A.to(dev), mod)
    torch.cuda.synchronize()
    tf, Af = f64(table), f64(A)
    want = np.zeros((L, len(conds), 2, hidden))
    bound = np.zeros_like(want)
    for l in range(L):
        for c, (nd, f) in enumerate(conds):
            t = tcond.t_cond(nd, f, tf)
            g, b = tcond.modulation(Af[l], t)
            want[l, c, 0], want[l, c, 1] = g, b
            # t_cond in float32: sin/cos rounded, then the table row added, so
            # |t'_i - t_i| <= 2^-24 (|e_i| + |t_i|); a float32 dot product over
            # D terms adds at most D 2^-24 sum_i |a_i t'_i|: together within
            # (D + 2) 2^-24 sum_i |a_i| (|t_i| + |e_i|)
            e = tcond.sinusoid(nd, dim)
            s = np.abs(Af[l]) @ (np.abs(t) + np.abs(e))
            bound[l, c, 0], bound[l, c, 1] = s[:hidden], s[hidden:]
    bound *= (dim + 2) * 2.0 ** -24
    return tc, mod, want, bound


def test_prepare_matches_the_oracle():
    rkv = rkv_mod()
    tc, mod, want, bound = _prepare(rkv, 3, 2048, 256, 41)
    err = np.abs(f64(mod) - want)
    say(f"prepare: max|err| {err.max():.3e}, max err/bound {(err / bound).max():.3f}")
    assert np.all(err <= bound)
    assert np.abs(want).max() > 0.05          # the vectors are not trivially small


@pytest.mark.parametrize("out_f32", [False, True])
def test_modulate_matches_the_oracle(out_f32):
    rkv = rkv_mod()
    dev = device()
    L, S, H, d = 3, 7, 16, 128
    flags = rkv.RKV_F_OUT_F32 if out_f32 else 0
    cfg = rkv.make_cfg(S, L, num_q_heads=H, num_kv_heads=2, head_dim=d, rebase_chunk=25,
                       flags=flags)
    tc, mod, want_mod, _ = _prepare(rkv, L, H * d, 256, 42)
    rng = np.random.default_rng(43)
    h = rng.standard_normal((L, S, H, d)).astype(np.float32)
    out = torch.from_numpy(h).to(dev)
    if not out_f32:
        out = out.to(torch.bfloat16)
    before = f64(out)
    cond = np.array([0, 7, -1, 3, 8, 5, 2], np.int32)     # -1: off; 8 = num_conds: off
    rkv.rkv_tcond_modulate(cfg, tc, mod, torch.from_numpy(cond).to(dev), out)
    torch.cuda.synchronize()
    got = f64(out).reshape(L, S, H * d)
    base = before.reshape(L, S, H * d)
    gm = f64(mod)
    for l in range(L):
        for s in range(S):
            c = cond[s]
            if c < 0 or c >= tc.num_conds:
                assert np.array_equal(got[l, s], base[l, s])
                continue
            if out_f32:
                # from the GPU's own vectors: one fma in float32
                w = base[l, s] * (1.0 + gm[l, c, 0]) + gm[l, c, 1]
                tol = 2.0 ** -23 * (np.abs(w) + np.abs(base[l, s])) + 1e-30
                assert np.all(np.abs(got[l, s] - w) <= tol)
                ref = tcond.modulate(base[l, s], want_mod[l, c, 0], want_mod[l, c, 1], None)
                assert np.abs(got[l, s] - ref).max() < 1e-4
            else:
                ref = tcond.modulate(base[l, s], want_mod[l, c, 0], want_mod[l, c, 1])
                assert np.all(np.abs(got[l, s] - ref) <= bf16_ulp(ref)), (l, s)
    say(f"modulate ({'f32' if out_f32 else 'bf16'} out): checked {L * S} rows")


def test_full_size_decode_step_output():
    """36 layers x 64 streams: one pipelined decode step, then the modulation
    of its output in place, every stream on one of the 8 settings or none."""
    rkv = rkv_mod()
    dev = device()
    L, S, W = 36, 64, 375
    cfg = rkv.make_cfg(S, L, rebase_chunk=25)
    cache = rkv.Cache(cfg, W, W, W, 0, device=dev)
    q, k, v = (x.to(dev) for x in synth.decoder_pool(44, L, S, 1, 16, 2, 128))
    out = torch.empty(q.shape[1:], dtype=torch.bfloat16, device=dev)
    rkv.rkv_advance(cfg, cache.state, cache.plan)
    rkv.rkv_decode_step_pipelined(cfg, cache.state, cache.plan, cache.plan_next, cache.kv, q[0],
                                  k[0], v[0], out, cache.workspace)
    tc, mod, want_mod, _ = _prepare(rkv, L, 2048, 256, 45)
    cond = (np.arange(S) % 9 - 1).astype(np.int32)
    base = f64(out).reshape(L, S, 2048)
    rkv.rkv_tcond_modulate(cfg, tc, mod, torch.from_numpy(cond).to(dev), out)
    torch.cuda.synchronize()
    got = f64(out).reshape(L, S, 2048)
    worst = 0.0
    for l in range(L):
        for s in range(S):
            c = cond[s]
            if c < 0:
                assert np.array_equal(got[l, s], base[l, s])
                continue
            ref = tcond.modulate(base[l, s], want_mod[l, c, 0], want_mod[l, c, 1])
            excess = np.abs(got[l, s] - ref) / bf16_ulp(ref)
            worst = max(worst, float(excess.max()))
    say(f"36 x 64 decode output modulated: worst |gpu - oracle| = {worst:.2f} bf16 ulp")
    assert worst <= 1.0


FUSED_CASES = [
    # name, mode, L, S, W, cap, splits, flags
    ("rebase", "rebase", 3, 5, 40, 40, 0, 0),
    ("rebase-f32", "rebase", 2, 5, 40, 40, 0, "f32"),
    ("split-in-launch", "rebase", 2, 3, 120, 120, 3, 0),
    ("split-merge-launch", "rebase", 2, 3, 120, 120, 3, "merge"),
    ("split-f32", "rebase", 1, 3, 120, 120, 4, "f32"),
    ("compact", "compact", 2, 3, 48, 64, 0, 0),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_fused_step_equals_step_then_modulate(case):
    """rkv_decode_step_pipelined_tcond against rkv_decode_step_pipelined +
    rkv_tcond_modulate on identical caches: every output bit and every ring
    byte the same, with streams on different conditions and some off (-1 and
    an index past the last condition), unsplit and split key ranges."""
    name, mode, L, S, W, cap, splits, flags = case
    rkv = rkv_mod()
    dev = device()
    fl = {0: 0, "f32": rkv.RKV_F_OUT_F32, "merge": rkv.RKV_F_MERGE_LAUNCH}[flags]
    md = rkv.RKV_MODE_REBASE if mode == "rebase" else rkv.RKV_MODE_COMPACT
    cfg = rkv.make_cfg(S, L, mode=md, rebase_chunk=5, flags=fl, num_splits=splits)
    hidden, C = 16 * 128, 4
    tc = rkv.make_tcond_cfg(L, hidden, dim=64, num_conds=C, max_frame_len=8)
    gen = torch.Generator().manual_seed(77)
    mod = (0.2 * torch.randn((L, C, 2, hidden), generator=gen)).to(dev)
    cond = torch.tensor([2, -1, 0, 3, C][:S], dtype=torch.int32, device=dev)
    T, P = 70, 16
    q = torch.randn((P, L, S, 16, 128), generator=gen).to(torch.bfloat16).to(dev)
    k = torch.randn((P, L, S, 2, 128), generator=gen).to(torch.bfloat16).to(dev)
    v = torch.randn((P, L, S, 2, 128), generator=gen).to(torch.bfloat16).to(dev)
    odt = torch.float32 if flags == "f32" else torch.bfloat16
    origins = np.arange(S, dtype=np.int64) * 7
    caches = [rkv.Cache(cfg, cap, W, cap, origins, device=dev) for _ in range(2)]
    outs = [torch.full((T, L, S, 16, 128), float("nan"), dtype=odt, device=dev) for _ in range(2)]
    say(f"case {name}: L={L} S={S} W={W} cap={cap} splits={splits or 'auto'} flags={flags}")
    for c in caches:
        rkv.rkv_advance(cfg, c.state, c.plan)
    for t in range(T):
        j = t % P
        for i, c in enumerate(caches):
            cur, nxt = (c.plan, c.plan_next) if t % 2 == 0 else (c.plan_next, c.plan)
            if md == rkv.RKV_MODE_COMPACT:
                rkv.rkv_compact(cfg, cur, c.kv)
            if i == 0:
                rkv.rkv_decode_step_pipelined(cfg, c.state, cur, nxt, c.kv, q[j], k[j], v[j],
                                              outs[0][t], c.workspace)
                rkv.rkv_tcond_modulate(cfg, tc, mod, cond, outs[0][t])
            else:
                rkv.rkv_decode_step_pipelined_tcond(cfg, tc, mod, cond, c.state, cur, nxt, c.kv,
                                                    q[j], k[j], v[j], outs[1][t], c.workspace)
    torch.cuda.synchronize()
    view = torch.int32 if odt == torch.float32 else torch.int16
    same = outs[0].view(view) == outs[1].view(view)
    say(f"  outputs identical: {int(same.sum())} of {same.numel()}")
    assert bool(torch.isfinite(outs[1].float()).all())
    assert bool(same.all())
    assert torch.equal(caches[0].buf.view(torch.int16), caches[1].buf.view(torch.int16))
