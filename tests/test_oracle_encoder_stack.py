"""Pins for oracle.encoder_stack: RMSNorm and GELU against closed forms and
library routines, and the layer step against a hand-unrolled single layer on
a tiny shape (brute force: explicit loops over heads and frames with the
attention written out), plus the residual structure with zero projections."""
import math

import numpy as np
import torch

from oracle import encoder_stack as es
from oracle import rope


def test_rmsnorm_and_gelu():
    x = np.array([[3.0, 4.0]])
    # mean of squares 12.5 -> x / sqrt(12.5)
    np.testing.assert_allclose(es.rmsnorm(x, np.ones(2), 0.0), x / math.sqrt(12.5), rtol=1e-15)
    y = np.linspace(-6, 6, 101)
    want = torch.nn.functional.gelu(torch.from_numpy(y), approximate="none").numpy()
    np.testing.assert_allclose(es.gelu(y), want, rtol=1e-12, atol=1e-15)
    assert es.gelu(0.0) == 0.0
    # the exact erf form, element by element with the standard library's erf
    z = np.random.default_rng(3).standard_normal(2000) * 3
    by_math = np.array([0.5 * t * (1.0 + math.erf(t / math.sqrt(2.0))) for t in z])
    # (1 + erf) cancels for large negative arguments: an absolute bound there
    np.testing.assert_allclose(es.gelu(z), by_math, rtol=1e-15, atol=1e-15)


def _weights(rng, hidden, ffn):
    m = lambda a, b: rng.standard_normal((a, b)) / math.sqrt(b)
    return dict(g1=1 + 0.1 * rng.standard_normal(hidden), wq=m(hidden, hidden),
                wk=m(hidden, hidden), wv=m(hidden, hidden), wo=m(hidden, hidden),
                g2=1 + 0.1 * rng.standard_normal(hidden), w1=m(ffn, hidden), w2=m(hidden, ffn))


def test_one_layer_against_hand_unrolled_steps():
    rng = np.random.default_rng(8)
    H, d, F, W, hidden, ffn, eps = 2, 4, 2, 3, 8, 16, 1e-5
    w = _weights(rng, hidden, ffn)
    st = es.EncoderStack([w], H, d, W, F, 1e6, eps, rounder=None)
    hist_k, hist_v = [], []                  # rotated K, V of every frame so far, per head
    for n in range(4):
        x = rng.standard_normal((F, hidden))
        got = st.step(x)
        a = x / np.sqrt((x ** 2).mean(axis=1, keepdims=True) + eps) * w["g1"]
        q, k, v = a @ w["wq"].T, a @ w["wk"].T, a @ w["wv"].T
        att = np.zeros((F, hidden))
        for j in range(F):
            pos = n * F + j
            hist_k.append([rope.rotate(k[j, h * d:(h + 1) * d], pos, 1e6) for h in range(H)])
            hist_v.append([v[j, h * d:(h + 1) * d] for h in range(H)])
        for j in range(F):
            pos = n * F + j
            lo = max(0, n * F - W)                      # the window before the chunk
            for h in range(H):
                qr = rope.rotate(q[j, h * d:(h + 1) * d], pos, 1e6)
                keys = [hist_k[p][h] for p in range(lo, pos + 1)]
                vals = [hist_v[p][h] for p in range(lo, pos + 1)]
                s = np.array([kk @ qr for kk in keys]) / math.sqrt(d)
                p = np.exp(s - s.max())
                p /= p.sum()
                att[j, h * d:(h + 1) * d] = sum(pi * vv for pi, vv in zip(p, vals))
        y = x + att @ w["wo"].T
        a2 = y / np.sqrt((y ** 2).mean(axis=1, keepdims=True) + eps) * w["g2"]
        hmid = a2 @ w["w1"].T
        u = 0.5 * hmid * (1 + np.vectorize(math.erf)(hmid / math.sqrt(2)))
        want = y + u @ w["w2"].T
        np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_zero_output_projections_leave_the_stream_unchanged():
    rng = np.random.default_rng(9)
    H, d, F, hidden = 2, 4, 2, 8
    w = _weights(rng, hidden, 32)
    w["wo"][:] = 0.0
    w["w2"][:] = 0.0
    st = es.EncoderStack([w, w], H, d, 6, F, 1e6, 1e-5)
    x = rng.standard_normal((F, hidden))
    np.testing.assert_array_equal(st.step(x), x)


def test_run_over_many_steps_equals_stepping():
    """run() (layer by layer over all steps) gives the values of step() called
    once per step, over enough steps to wrap a ring whose size is not a
    multiple of the chunk, with bfloat16 storage points."""
    rng = np.random.default_rng(10)
    H, d, F, W, hidden, ffn, T = 2, 8, 4, 10, 16, 32, 9      # ring of 14 slots
    ws = [_weights(rng, hidden, ffn) for _ in range(2)]
    xs = rng.standard_normal((T, F, hidden))
    a = es.EncoderStack(ws, H, d, W, F, 1e6, 1e-5)
    b = es.EncoderStack(ws, H, d, W, F, 1e6, 1e-5)
    stepped = np.stack([a.step(x) for x in xs])
    np.testing.assert_allclose(b.run(xs), stepped, rtol=1e-12, atol=1e-12)
