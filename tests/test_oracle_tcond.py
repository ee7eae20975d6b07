"""Pins for oracle.tcond: the delay-token count against the model card's
table of post-trained delays and the explainer's worked example (480 ms at
80 ms -> 6), the sinusoidal embedding against hand-worked values and the
angle-addition identity, and the feature-wise modulation against a
hand-worked example and brute force."""
import json
import os

import numpy as np
import pytest

from oracle import tcond
from oracle.bf16 import round_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


def golden():
    return json.load(open(GOLDEN))


def test_delay_tokens_over_the_post_trained_table():
    g = golden()
    frame_len = {c["clock_ms"]: c["frame_len"] for c in g["clocks"]["value"]}
    want = {80: [3, 4, 6, 7], 120: [2, 4], 160: [2, 3]}
    for clock, delays in g["post_trained_delays_ms"]["value"].items():
        got = [tcond.delay_tokens(d, int(clock)) for d in delays]
        assert [n for n, _ in got] == want[int(clock)]
        assert all(f == frame_len[int(clock)] for _, f in got)
    assert tcond.delay_tokens(480, 80)[0] == g["num_delay_tokens_480ms_80ms"]["value"]
    # longer delays stay available at every clock (integer multiples)
    assert tcond.delay_tokens(1600, 160) == (10, 8)


@pytest.mark.parametrize("delay,clock", [(500, 80), (240, 160), (320, 120), (0, 80),
                                         (-80, 80), (480, 100), (480, 40)])
def test_delay_tokens_rejects_illegal_settings(delay, clock):
    with pytest.raises(ValueError):
        tcond.delay_tokens(delay, clock)


def test_sinusoid_hand_values():
    # D = 4: frequencies 1 and 10000^(-1/2) = 0.01
    np.testing.assert_allclose(tcond.sinusoid(6, 4),
                               [-0.27941549819892586, 0.059964006479444595,
                                0.960170286650366, 0.9982005399352042], rtol=0, atol=1e-15)
    # D = 6: frequencies 1, 10000^(-1/3), 10000^(-2/3)
    np.testing.assert_allclose(tcond.sinusoid(3, 6),
                               [0.1411200080598672, 0.13879810108005053, 0.006463259070189645,
                                -0.9899924966004454, 0.990320699135675, 0.9999791129229608],
                               rtol=0, atol=1e-15)


def test_sinusoid_identities():
    D = 256
    h = D // 2
    e0 = tcond.sinusoid(0, D)
    assert np.array_equal(e0, np.concatenate([np.zeros(h), np.ones(h)]))
    for n in (1, 6, 37):
        e = tcond.sinusoid(n, D)
        np.testing.assert_allclose(e[:h] ** 2 + e[h:] ** 2, 1.0, atol=1e-15)
    # angle addition: cos + i sin of (n + m) is the product of those of n and m
    z = lambda n: (lambda e: e[h:] + 1j * e[:h])(tcond.sinusoid(n, D))
    np.testing.assert_allclose(z(9), z(4) * z(5), atol=1e-14)
    # frequencies fall geometrically from 1 by 10000^(1/h) per index
    e1 = tcond.sinusoid(1, D)
    w = np.arctan2(e1[:h], e1[h:])
    assert w[0] == pytest.approx(1.0)
    np.testing.assert_allclose(w[1:] / w[:-1], 10000.0 ** (-1.0 / h), rtol=1e-12)
    with pytest.raises(ValueError):
        tcond.sinusoid(1, 5)


def test_t_cond_adds_the_frame_length_row():
    table = np.array([[0.0, 0.0, 0.0, 0.0], [1.0, -1.0, 0.5, 2.0], [0.25, 0.25, 0.25, 0.25]])
    got = tcond.t_cond(6, 1, table)
    np.testing.assert_allclose(got, [-0.27941549819892586 + 1.0, 0.059964006479444595 - 1.0,
                                     0.960170286650366 + 0.5, 0.9982005399352042 + 2.0],
                               atol=1e-15)


def test_modulate_hand_example():
    h = np.array([1.0, 2.0, -3.0, 0.5])
    gamma = np.array([0.5, -1.0, 0.0, 1.0])
    beta = np.array([0.25, 3.0, -1.0, 0.0])
    assert np.array_equal(tcond.modulate(h, gamma, beta), [1.75, 3.0, -4.0, 1.0])
    # rounding to bfloat16 after the modulation: 1 + 2^-9 is not representable
    assert tcond.modulate(np.array([1.0]), np.array([2.0 ** -9]), np.array([0.0]))[0] == 1.0


def test_modulation_against_brute_force():
    rng = np.random.default_rng(5)
    H, D = 6, 8
    A = rng.standard_normal((2 * H, D))
    tc = rng.standard_normal(D)
    gamma, beta = tcond.modulation(A, tc)
    for j in range(H):
        s_g = 0.0
        s_b = 0.0
        for i in range(D):
            s_g += A[j, i] * tc[i]
            s_b += A[H + j, i] * tc[i]
        assert gamma[j] == pytest.approx(s_g, abs=1e-12)
        assert beta[j] == pytest.approx(s_b, abs=1e-12)
    h = round_bf16(rng.standard_normal((3, H)))
    zg, zb = tcond.modulation(np.zeros((2 * H, D)), tc)
    assert np.array_equal(tcond.modulate(h, zg, zb), h)        # zero weights: identity
