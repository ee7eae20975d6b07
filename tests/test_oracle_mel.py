"""Pins for oracle.mel (the rolling log-mel front end): the Slaney scale's
closed forms, filter areas and peaks, the real DFT against a brute-force sum,
a pure tone landing in the filter whose band holds it, and the rolling buffer
(only the n_fft - hop newest samples kept) giving exactly the frames of the
whole signal."""
import numpy as np
import pytest

from oracle import mel


def test_slaney_scale_closed_forms():
    assert mel.hz_to_mel(0.0) == 0.0
    assert mel.hz_to_mel(200.0 / 3.0) == pytest.approx(1.0, abs=1e-12)
    assert mel.hz_to_mel(1000.0) == pytest.approx(15.0, abs=1e-12)
    assert mel.hz_to_mel(6400.0) == pytest.approx(42.0, abs=1e-12)   # 1 kHz x 6.4 = 27 steps up
    f = np.array([10.0, 500.0, 999.0, 1000.0, 1500.0, 8000.0])
    np.testing.assert_allclose(mel.mel_to_hz(mel.hz_to_mel(f)), f, rtol=1e-12)


def test_filters_are_unit_area_triangles():
    w = mel.mel_filters()
    assert w.shape == (128, 201)
    assert np.all(w >= 0)
    df = mel.SAMPLE_RATE / mel.N_FFT                 # 40 Hz per bin
    edges = mel.mel_to_hz(np.linspace(0.0, mel.hz_to_mel(8000.0), 130))
    for m in range(128):
        width = edges[m + 2] - edges[m]
        if width > 12 * df:                          # well resolved by the bins
            assert np.sum(w[m]) * df == pytest.approx(1.0, rel=0.05)
        if np.any(w[m] > 0):
            peak_hz = np.argmax(w[m]) * df
            assert abs(peak_hz - edges[m + 1]) <= df


def test_dft_matches_brute_force_sum():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 400))
    wnd = np.array([0.5 - 0.5 * np.cos(2 * np.pi * n / 400) for n in range(400)])
    k = np.arange(201)[:, None]
    n = np.arange(400)[None, :]
    re = (x * wnd) @ np.cos(2 * np.pi * k * n / 400).T
    im = -(x * wnd) @ np.sin(2 * np.pi * k * n / 400).T
    energy = re ** 2 + im ** 2
    want = np.log10(np.maximum(energy @ mel.mel_filters().T, 1e-10))
    np.testing.assert_allclose(mel.log_mel_frames(x), want, rtol=0, atol=1e-9)
    assert mel.hann()[0] == 0.0 and mel.hann()[200] == 1.0
    np.testing.assert_allclose(mel.hann()[1:], mel.hann()[1:][::-1], atol=1e-15)


@pytest.mark.parametrize("f0", [440.0, 1000.0, 3000.0, 6000.0])
def test_pure_tone_lands_in_its_band(f0):
    t = np.arange(16000) / 16000.0
    frames = mel.whole_signal(np.sin(2 * np.pi * f0 * t))
    peak = np.argmax(frames[10:].mean(axis=0))
    edges = mel.mel_to_hz(np.linspace(0.0, mel.hz_to_mel(8000.0), 130))
    # the filter with the strongest response is one whose band contains f0
    assert edges[peak] < f0 < edges[peak + 2]


def test_rolling_buffer_equals_whole_signal():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(1280 * 9) * 0.1
    roll = mel.RollingMel()
    got = np.concatenate([roll.step(x[i:i + 1280]) for i in range(0, x.size, 1280)])
    want = mel.whole_signal(x)
    assert got.shape == (72, 128) and want.shape == (72, 128)
    # the same frames; batched FFTs of different batch sizes may differ in
    # the last bit, a wrong buffer would differ by O(1)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    assert roll.tail.size == 240
    np.testing.assert_array_equal(roll.tail, x[-240:])


def test_first_frames_see_zeros_before_the_stream():
    # frame 0 covers 240 zeros and the first 160 samples: a stream of silence
    # then a click at sample 0 shows the click in frame 0 and frame 1 only
    x = np.zeros(1280)
    x[0] = 1.0
    frames = mel.whole_signal(x)
    assert frames[0].max() > -9 and frames[1].max() > -9
    assert np.all(frames[3:] == np.log10(1e-10))
