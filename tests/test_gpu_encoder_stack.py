"""rkv_encoder_step (the incremental encoder step through a stack of layers
around the chunk attention) against the float64 oracle with bfloat16 storage
points (oracle.encoder_stack).

Every case is checked two ways:

* layer by layer (teacher forced): each layer's GPU output against the oracle
  layer fed the GPU's own input of that layer, over every step (the oracle
  layer's ring is built from those inputs), within GATE;
* end to end: the stack's output against the oracle stack fed the frame
  embeddings.  A one-ulp bfloat16 rounding flip in a stored activation of one
  layer feeds every later layer, so two correct computations drift apart with
  depth even though each layer agrees within GATE.  The bound is measured,
  not guessed: the test runs the oracle stack a second and third time with
  every stored value perturbed by a relative 2^-16 (about the float32
  accumulation error of the GPU's sums and its 16-bit softmax weights) before
  its bfloat16 rounding, and takes the largest distance between those runs
  and the plain oracle as the spread of equally valid results; the GPU must
  stay within twice that spread.

The cases run past the window fill and through ring wraps, with a ring size
that is not a multiple of the chunk (chunks straddle the wrap); the full
32-layer, 128-stream, hidden 1280 case also checks that the one 32-layer call
equals 32 one-layer calls bit for bit at every step."""
import numpy as np
import pytest
import torch

from oracle import encoder_stack as oes
from oracle.bf16 import round_bf16
from rolling_window_kv_amd import synth

from gpu_util import device, rkv_mod, say

pytestmark = pytest.mark.gpu

GATE = 2e-2          # max |gpu - oracle| / max(1, rms(oracle)) of one layer's output
PERTURB = 2.0 ** -16  # relative perturbation of the stored values in the spread runs


def _err(got, want):
    """max |got - want| / max(1, rms(want)) over the last two axes, per step."""
    rms = np.sqrt((want ** 2).mean(axis=(-2, -1)))
    return np.abs(got - want).max(axis=(-2, -1)) / np.maximum(1.0, rms)


def _perturbed_rounder(seed):
    rng = np.random.default_rng(seed)

    def rounder(x):
        x = np.asarray(x, np.float64)
        return round_bf16(x * (1.0 + PERTURB * rng.uniform(-1.0, 1.0, x.shape)))
    return rounder


def _cfg(rkv, L, S, H, d, F):
    return rkv.make_cfg(S, L, num_q_heads=H, num_kv_heads=H, head_dim=d,
                        mode=rkv.RKV_MODE_ENC_CHUNK, new_rows=F)


def _run_gpu(rkv, L, S, H, d, F, W, ffn, seed, steps, check):
    """Drive the stack on the GPU twice from the same embeddings: one L-layer
    call per step, and L one-layer calls per step with their own caches.
    Returns the embeddings and, for the checked streams, every layer's input
    and output per step ([steps, L + 1, F, hidden] float64: index 0 is the
    stack input, index l + 1 the output of layer l)."""
    dev = device()
    hidden = H * d
    cap = W + F
    ecfg = rkv.make_encoder_cfg(ffn=ffn, norm_eps=1e-5)
    layers = synth.encoder_stack_weights(seed, L, hidden, ffn)
    xin = synth.encoder_stack_inputs(seed, S, steps, F, hidden)
    cfg = _cfg(rkv, L, S, H, d, F)
    cfg1 = _cfg(rkv, 1, S, H, d, F)
    fused = rkv.Cache(cfg, cap, W, cap, 0, device=dev)
    per = [rkv.Cache(cfg1, cap, W, cap, 0, device=dev) for _ in range(L)]
    wdev = rkv.pack_encoder_weights(layers).to(dev)
    lw = rkv.rkv_encoder_layer_weight_bytes(cfg, ecfg) // 2
    assert wdev.numel() == L * lw
    ws = torch.empty(rkv.rkv_encoder_step_workspace_bytes(cfg, ecfg, cap), dtype=torch.uint8,
                     device=dev)
    idx = torch.tensor(check, device=dev)
    trace = np.zeros((len(check), steps, L + 1, F, hidden))
    for t in range(steps):
        xf = xin[t].to(dev).contiguous()
        rkv.rkv_advance(cfg, fused.state, fused.plan)
        rkv.rkv_encoder_step(cfg, ecfg, fused.plan, fused.kv, wdev, xf, ws)
        xl = xin[t].to(dev).contiguous()
        snaps = [xl.index_select(0, idx)]
        for l, c in enumerate(per):
            rkv.rkv_advance(cfg1, c.state, c.plan)
            rkv.rkv_encoder_step(cfg1, ecfg, c.plan, c.kv, wdev[l * lw:(l + 1) * lw], xl, ws)
            snaps.append(xl.index_select(0, idx))
        assert torch.equal(xf, xl), f"step {t}: the {L}-layer call != {L} one-layer calls"
        trace[:, t] = torch.stack(snaps, 1).cpu().numpy()
    wts = [{n: t.double().numpy() for n, t in lw_.items()} for lw_ in layers]
    return xin, wts, trace


def _check(L, H, d, F, W, xin, wts, trace, check, end_to_end):
    """Teacher-forced layer gate for every checked stream; end-to-end gate for
    the streams in `end_to_end`."""
    worst_layer = 0.0
    for i, s in enumerate(check):
        for l in range(L):
            want = oes.EncoderStack([wts[l]], H, d, W, F, 1e6, 1e-5).run(trace[i, :, l])
            e = float(_err(trace[i, :, l + 1], want).max())
            worst_layer = max(worst_layer, e)
            if l % 8 == 7:
                say(f"stream {s}: oracle layers 0..{l} done, worst {worst_layer:.3e}")
        say(f"stream {s}: worst teacher-forced layer {worst_layer:.3e} (gate {GATE:g})")
    assert worst_layer < GATE
    for i, s in enumerate(check):
        if s not in end_to_end:
            continue
        x = xin[:, s].double().numpy()
        want = oes.EncoderStack(wts, H, d, W, F, 1e6, 1e-5).run(x)
        say(f"stream {s}: oracle stack done")
        spread = 0.0
        for seed in (1, 2):
            pert = oes.EncoderStack(wts, H, d, W, F, 1e6, 1e-5,
                                    rounder=_perturbed_rounder(seed)).run(x)
            spread = max(spread, float(_err(pert, want).max()))
            say(f"stream {s}: perturbed oracle run {seed} done")
        got = float(_err(trace[i, :, L], want).max())
        say(f"stream {s}: end to end max |gpu - oracle| / max(1, rms) {got:.3e}; "
            f"spread of the perturbed oracle runs {spread:.3e}; gate {2 * spread:.3e}")
        assert got <= 2.0 * spread


@pytest.mark.timeout(300)
@pytest.mark.parametrize("L,S,H,ffn,steps", [(3, 3, 4, 1024, 24), (2, 3, 5, 640, 20)])
def test_small_stack_wraps_the_ring(L, S, H, ffn, steps):
    """3 streams x 4 frames = 12 tokens (a ragged tile), window 30 frames in a
    34-slot ring (34 = 8 chunks + 2 slots: chunks straddle the wrap), full from
    step 8 on and wrapped twice; hidden 256 / MLP 1024 (both residual products
    in four k-slices) and hidden 320 / MLP 640 (the output projection in one
    slice, the MLP's second product in two)."""
    rkv = rkv_mod()
    d, F, W = 64, 4, 30
    check = tuple(range(S))
    say(f"small stack: L={L} S={S} H={H} ffn={ffn} steps={steps}")
    xin, wts, trace = _run_gpu(rkv, L, S, H, d, F, W, ffn, 77, steps, check)
    _check(L, H, d, F, W, xin, wts, trace, check, end_to_end=check)


@pytest.mark.timeout(1200)     # the float64 oracle of 192 steps x 32 layers takes minutes
def test_full_shape_32_layers_128_streams():
    """The encoder workload's shape (32 layers, 128 streams, hidden 1280 as
    20 x 64, MLP 5120, window 750 in a 754-slot ring) for 192 steps: the
    window fills at step 188 and the ring wraps at step 189, in the middle of
    a chunk."""
    rkv = rkv_mod()
    L, S, H, d, F, W, ffn, steps = 32, 128, 20, 64, 4, 750, 5120, 192
    check = (0, 127)
    say(f"full stack: L={L} S={S} steps={steps}")
    xin, wts, trace = _run_gpu(rkv, L, S, H, d, F, W, ffn, 78, steps, check)
    _check(L, H, d, F, W, xin, wts, trace, check, end_to_end=(0,))
