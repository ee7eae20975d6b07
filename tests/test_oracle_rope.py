"""Pins for oracle.rope: closed-form frequencies, a hand-computed rotation,
the complex-number form of RoPE, and the group identities the method relies on
(R(-D) R(p) = R(p - D) is what makes re-basing exact)."""
import math

import numpy as np

from oracle import rope


def test_frequencies_closed_form():
    th = rope.inv_freq(128, 1e6)
    assert th.shape == (64,)
    assert th[0] == 1.0
    assert abs(th[32] - 1e-3) < 1e-18            # 1e6 ** (-64/128)
    np.testing.assert_allclose(th[1:] / th[:-1], 1e6 ** (-2 / 128), rtol=1e-13)


def test_hand_example():
    # d = 4, base 100: theta = [1, 0.1]; pairs (x0, x2) and (x1, x3).
    x = np.array([1.0, 2.0, 3.0, 4.0])
    p = math.pi / 2
    y = rope.rotate(x, p, 100.0)
    a1 = 0.1 * p
    want = [1 * math.cos(p) - 3 * math.sin(p),
            2 * math.cos(a1) - 4 * math.sin(a1),
            1 * math.sin(p) + 3 * math.cos(p),
            2 * math.sin(a1) + 4 * math.cos(a1)]
    np.testing.assert_allclose(y, want, atol=1e-15)
    assert abs(y[0] + 3.0) < 1e-15 and abs(y[2] - 1.0) < 1e-15


def test_complex_form():
    rng = np.random.default_rng(0)
    d = 128
    x = rng.standard_normal((5, d))
    pos = np.array([0, 1, 17, 375, 20000])
    z = (x[:, : d // 2] + 1j * x[:, d // 2:]) * np.exp(
        1j * pos[:, None] * (1e6 ** (-np.arange(0, d, 2) / d)))
    y = rope.rotate(x, pos, 1e6)
    np.testing.assert_allclose(y[:, : d // 2], z.real, atol=1e-12)
    np.testing.assert_allclose(y[:, d // 2:], z.imag, atol=1e-12)


def test_group_identities():
    d, base = 128, 1e6
    r = lambda p: rope.rotation_matrix(p, d, base)
    np.testing.assert_allclose(r(0), np.eye(d), atol=1e-15)
    for a, b in [(3, 5), (374, -25), (10000, -9999), (-1, 1)]:
        np.testing.assert_allclose(r(a) @ r(b), r(a + b), atol=1e-12)
    m = r(123.0)
    np.testing.assert_allclose(m @ m.T, np.eye(d), atol=1e-12)
    assert abs(np.linalg.det(m) - 1.0) < 1e-10
    rng = np.random.default_rng(3)
    x = rng.standard_normal(d)
    for p, delta in [(399, 25), (374, 1), (9000, 1024)]:
        np.testing.assert_allclose(rope.rotate(rope.rotate(x, p, base), -delta, base),
                                   rope.rotate(x, p - delta, base), atol=1e-12)


def test_relative_position_property():
    rng = np.random.default_rng(4)
    d, base = 64, 1e6
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for m, n in [(10, 3), (400, 26), (12345, 12000)]:
        lhs = rope.rotate(q, m, base) @ rope.rotate(k, n, base)
        rhs = rope.rotate(q, m - n, base) @ k
        assert abs(lhs - rhs) < 1e-10
