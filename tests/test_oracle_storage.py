"""Pins for oracle.storage: without rounding, the step-by-step ring, buffer and
encoder simulations must equal the exact oracle (this checks the re-base,
compaction and slot logic through RoPE's shift invariance); with bfloat16
rounding the error stays small, and compensation removes the drift that plain
re-rounding shows at one re-base per step."""
import numpy as np
import pytest

from oracle import attention as att
from oracle import rope
from oracle import storage as stg
from oracle.bf16 import round_bf16


def _seq(T, hq, hkv, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, hq, d)), rng.standard_normal((T, hkv, d)),
            rng.standard_normal((T, hkv, d)))


@pytest.mark.parametrize("W,dc,origin,comp", [(6, 1, 0, False), (6, 1, 3, True), (7, 3, 5, False), (9, 4, 0, True)])
def test_rebase_ring_unrounded_equals_exact(W, dc, origin, comp):
    T, hq, hkv, d = 40, 4, 2, 16
    q, k, v = _seq(T, hq, hkv, d, 10)
    ring = stg.RebaseRing(hq, hkv, d, W, dc, 1e6, origin, comp, rounder=None)
    exact = att.window_decode(q, k, v, W, 1e6, origin)
    for t in range(T):
        _, out = ring.step(q[t], k[t], v[t])
        np.testing.assert_allclose(out, exact[t], atol=1e-10)


def test_compact_buffer_unrounded_equals_exact():
    T, hq, hkv, d = 45, 4, 2, 8
    q, k, v = _seq(T, hq, hkv, d, 11)
    buf = stg.CompactBuffer(hq, hkv, d, 5, 8, 1e6, origin=17, rounder=None)
    exact = att.compact_decode(q, k, v, 5, 8, 1e6, origin=17)
    for t in range(T):
        _, out = buf.step(q[t], k[t], v[t])
        np.testing.assert_allclose(out, exact[t], atol=1e-10)


def test_encoder_ring_unrounded_equals_exact():
    n, F, H, d, W = 12, 4, 2, 8, 9
    rng = np.random.default_rng(12)
    q, k, v = (rng.standard_normal((n, F, H, d)) for _ in range(3))
    ring = stg.EncoderRing(H, d, W, F, 1e6, origin=6, rounder=None)
    exact = att.encoder_chunks(q, k, v, W, 1e6, origin=6)
    for c in range(n):
        _, out = ring.step(q[c], k[c], v[c])
        np.testing.assert_allclose(out, exact[c], atol=1e-10)


def test_rebase_calls_compose_without_rounding():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((3, 128))
    hi, lo = stg.append_k(x, 400, 1e6, rounder=None)
    h1, l1 = stg.rebase_k(hi, lo, 25, 1e6, rounder=None)
    h2, l2 = stg.rebase_k(h1, l1, 25, 1e6, rounder=None)
    np.testing.assert_allclose(h2, rope.rotate(x, 350, 1e6), atol=1e-12)


def test_compensated_pair_carries_the_residual():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((64, 128))
    hi, lo = stg.append_k(x, 300, 1e6, compensated=True)
    y = rope.rotate(x, 300, 1e6)
    np.testing.assert_array_equal(hi, round_bf16(y))
    assert np.max(np.abs(hi + lo - y)) <= np.max(np.abs(y)) * 2.0 ** -16


def test_plain_rerounding_stalls_slow_pairs():
    # A slow pair of two unit components rotated by one step per call never
    # moves once rounded: theta_40 (about 1.8e-4) is below half a bfloat16 ulp
    # of 1.  The compensated pair follows the exact rotation.
    d, base = 128, 1e6
    k = np.zeros(d)
    k[40], k[40 + 64] = 1.0, 1.0
    hi, _ = stg.append_k(k, 0, base)
    x = hi
    for _ in range(100):
        x, _ = stg.rebase_k(x, 0 * x, 1, base)
    np.testing.assert_array_equal(x, hi)
    xh, xl = stg.append_k(k, 0, base, compensated=True)
    for _ in range(100):
        xh, xl = stg.rebase_k(xh, xl, 1, base, compensated=True)
    exact = rope.rotate(k, -100, base)
    assert np.max(np.abs((xh + xl) - exact)) < 2.0 ** -12
    assert np.max(np.abs(hi - exact)) > 0.01


def test_bf16_storage_error_small_for_chunked_rebase():
    T, W, dc = 160, 50, 5
    q, k, v = _seq(T, 8, 1, 128, 15)
    q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    ring = stg.RebaseRing(8, 1, 128, W, dc, 1e6)
    exact = att.window_decode(q, k, v, W, 1e6)
    err = 0.0
    for t in range(T):
        _, out = ring.step(q[t], k[t], v[t])
        err = max(err, np.max(np.abs(out - exact[t])))
    assert err < 2e-2


def test_fp16_storage_rounds_k_and_v_in_binary16():
    # fp16 cache variant (voxtral.c explainer, section 七): every stored K and
    # V is a binary16 value; a V input below the binary16 normal range is
    # rounded to its subnormal grid, and K after the append is the binary16
    # rounding of the exact rotation.
    from oracle import fp16, rope
    rng = np.random.default_rng(12)
    ring = stg.RebaseRing(2, 1, 8, 4, 2, 1e6, rounder=fp16.round_f16)
    k = rng.standard_normal((1, 8))
    v = np.full((1, 8), 1.0e-6)
    q = rng.standard_normal((2, 8))
    plan, _ = ring.step(q, k, v)
    assert np.all(ring.v[0, plan.slot] == fp16.round_f16(1.0e-6))
    assert np.all(ring.v[0, plan.slot] != 1.0e-6)
    np.testing.assert_array_equal(ring.k_hi[0, plan.slot],
                                  fp16.round_f16(rope.rotate(k, plan.pos, 1e6))[0])
