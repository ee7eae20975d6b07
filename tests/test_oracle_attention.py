"""Pins for oracle.attention: a scalar brute force written from the definition,
PyTorch's scaled_dot_product_attention (a library routine) for the
window-covers-everything case, and the degenerate cases of the method."""
import math

import numpy as np
import torch

from oracle import attention as att
from oracle import rope


def brute_force_decode(q, k, v, window, base, origin):
    """Triple loop in plain Python floats: rotate, dot, softmax, weighted sum."""
    T, hq, d = q.shape
    hkv = k.shape[1]
    half = d // 2

    def rot(x, p):
        y = [0.0] * d
        for i in range(half):
            ang = p * base ** (-2.0 * i / d)
            c, s = math.cos(ang), math.sin(ang)
            y[i] = x[i] * c - x[i + half] * s
            y[i + half] = x[i] * s + x[i + half] * c
        return y

    out = np.zeros((T, hq, d))
    for t in range(T):
        keys = list(range(max(0, t - window + 1), t + 1))
        for h in range(hq):
            g = h * hkv // hq
            qr = rot(list(q[t, h]), origin + t)
            scores = []
            for j in keys:
                kr = rot(list(k[j, g]), origin + j)
                scores.append(sum(a * b for a, b in zip(qr, kr)) / math.sqrt(d))
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            tot = sum(w)
            for e in range(d):
                out[t, h, e] = sum(w[n] * v[keys[n], g, e] for n in range(len(keys))) / tot
    return out


def _inputs(T, hq, hkv, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, hq, d)), rng.standard_normal((T, hkv, d)),
            rng.standard_normal((T, hkv, d)))


def test_brute_force_small():
    q, k, v = _inputs(12, 4, 2, 8, 0)
    got = att.window_decode(q, k, v, window=4, base=10000.0, origin=5)
    want = brute_force_decode(q, k, v, 4, 10000.0, 5)
    for t in range(12):
        np.testing.assert_allclose(got[t], want[t], atol=1e-12)


def test_window_covering_history_is_causal_sdpa():
    q, k, v = _inputs(20, 8, 2, 16, 1)
    base = 1e6
    got = att.window_decode(q, k, v, window=1000, base=base)
    pos = np.arange(20)
    qr = torch.from_numpy(rope.rotate(q, pos[:, None], base)).permute(1, 0, 2)
    kr = torch.from_numpy(rope.rotate(k, pos[:, None], base)).permute(1, 0, 2)
    vt = torch.from_numpy(v).permute(1, 0, 2)
    kr = kr.repeat_interleave(4, dim=0)
    vt = vt.repeat_interleave(4, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qr[None], kr[None], vt[None], is_causal=True)[0].permute(1, 0, 2).numpy()
    for t in range(20):
        np.testing.assert_allclose(got[t], ref[t], atol=1e-12)


def test_window_one_returns_current_value():
    q, k, v = _inputs(10, 4, 2, 8, 2)
    got = att.window_decode(q, k, v, window=1, base=1e6)
    for t in range(10):
        np.testing.assert_allclose(got[t], np.repeat(v[t], 2, axis=0), atol=1e-15)


def test_zero_query_averages_window():
    q, k, v = _inputs(30, 4, 2, 8, 3)
    q[:] = 0.0
    got = att.window_decode(q, k, v, window=7, base=1e6)
    for t in range(30):
        lo = max(0, t - 6)
        np.testing.assert_allclose(got[t], np.repeat(v[lo:t + 1].mean(0), 2, axis=0),
                                   atol=1e-14)


def test_gqa_equals_mha_with_repeated_kv():
    q, k, v = _inputs(15, 8, 2, 8, 4)
    gqa = att.window_decode(q, k, v, window=5, base=1e6)
    mha = att.window_decode(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1),
                            window=5, base=1e6)
    for t in range(15):
        np.testing.assert_allclose(gqa[t], mha[t], atol=1e-14)


def test_shift_invariance_of_absolute_positions():
    q, k, v = _inputs(25, 4, 2, 16, 5)
    a = att.window_decode(q, k, v, window=6, base=1e6, origin=0)
    b = att.window_decode(q, k, v, window=6, base=1e6, origin=1_000_003)
    for t in range(25):
        np.testing.assert_allclose(a[t], b[t], atol=1e-10)


def test_compaction_without_overflow_is_causal():
    q, k, v = _inputs(18, 4, 2, 8, 6)
    a = att.compact_decode(q, k, v, window=4, cap=100, base=1e6)
    b = att.window_decode(q, k, v, window=10 ** 6, base=1e6)
    for t in range(18):
        np.testing.assert_allclose(a[t], b[t], atol=1e-14)


def test_compaction_attends_retained_rows():
    # window 3, cap 5: rows retained at step t are [t - len + 1, t].
    q, k, v = _inputs(14, 2, 1, 8, 7)
    got = att.compact_decode(q, k, v, window=3, cap=5, base=1e6)
    lens = [1, 2, 3, 4, 5, 4, 5, 4, 5, 4, 5, 4, 5, 4]
    for t in range(14):
        want = att.attend_history(q, k, v, [t - lens[t] + 1] * 14, 1e6, steps=[t])[t]
        np.testing.assert_allclose(got[t], want, atol=1e-14)


def test_encoder_single_frame_is_window_decode():
    # F = 1: frame P attends [P - W, P], i.e. a window of W + 1 tokens, MHA.
    rng = np.random.default_rng(8)
    n, H, d, W = 20, 3, 8, 5
    q, k, v = (rng.standard_normal((n, 1, H, d)) for _ in range(3))
    enc = att.encoder_chunks(q, k, v, window=W, base=1e6, origin=2)
    dec = att.window_decode(q[:, 0], k[:, 0], v[:, 0], window=W + 1, base=1e6, origin=2)
    for t in range(n):
        np.testing.assert_allclose(enc[t][0], dec[t], atol=1e-13)


def test_encoder_chunk_brute_force():
    rng = np.random.default_rng(9)
    n, F, H, d, W = 6, 4, 2, 8, 7
    q, k, v = (rng.standard_normal((n, F, H, d)) for _ in range(3))
    got = att.encoder_chunks(q, k, v, window=W, base=100.0)
    fq, fk, fv = (x.reshape(n * F, H, d) for x in (q, k, v))
    for c in range(n):
        P = c * F
        for j in range(F):
            lo = max(0, P - W)
            for h in range(H):
                qr = rope.rotate(fq[P + j, h], P + j, 100.0)
                s = np.array([qr @ rope.rotate(fk[m, h], m, 100.0) for m in range(lo, P + j + 1)])
                w = np.exp(s / math.sqrt(d) - (s / math.sqrt(d)).max())
                ref = (w[:, None] * fv[lo:P + j + 1, h]).sum(0) / w.sum()
                np.testing.assert_allclose(got[c][j, h], ref, atol=1e-13)
