"""Rolling log-mel front end (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring): float64 NumPy.

voxtral.c explainer, section 三: even the mel-spectrogram buffer rolls -- old
audio samples that can no longer contribute to any future mel frame are
dropped (mel_compact_samples), so every stage of the pipeline has bounded
memory.  The Audio8 explainer's file table gives the features: 16 kHz audio,
128 mel bands, hop 160 samples (10 ms); a decoder step of the 80 ms clock
carries 1280 samples (8 hops).

Readings taken where the pages give no detail:

  * analysis window n_fft = 400 samples (25 ms), periodic Hann window
    w[n] = 0.5 - 0.5 cos(2 pi n / n_fft), real DFT bins k = 0 .. n_fft / 2;
  * frames are causal: frame f covers samples [f*hop - (n_fft - hop),
    f*hop + hop), the stream starting with n_fft - hop zero samples, so each
    step of S samples yields exactly S / hop new frames and a frame never
    waits for future audio;
  * the rolling buffer keeps exactly the n_fft - hop newest samples between
    steps: every older sample lies before the start of every future frame;
  * mel filterbank: the Slaney mel scale (linear below 1 kHz, logarithmic
    above) with triangular filters between 0 Hz and the Nyquist frequency
    and area normalisation (each triangle scaled by 2 / its width in Hz);
  * features: log10(max(mel energy, 1e-10)), energy = |X_k|^2.
"""
from __future__ import annotations

import numpy as np

SAMPLE_RATE = 16000
N_FFT = 400
HOP = 160
N_MELS = 128
SAMPLES_PER_STEP = 1280
LOG_FLOOR = 1e-10

# Slaney mel scale: 3 mel per 200 Hz below 1 kHz, then a constant ratio per
# mel step (6.4 over 27 mel steps).
_F_SP = 200.0 / 3.0
_MIN_LOG_HZ = 1000.0
_MIN_LOG_MEL = _MIN_LOG_HZ / _F_SP
_LOGSTEP = np.log(6.4) / 27.0


def hz_to_mel(f):
    f = np.asarray(f, np.float64)
    lin = f / _F_SP
    log = _MIN_LOG_MEL + np.log(np.maximum(f, _MIN_LOG_HZ) / _MIN_LOG_HZ) / _LOGSTEP
    return np.where(f >= _MIN_LOG_HZ, log, lin)


def mel_to_hz(m):
    m = np.asarray(m, np.float64)
    lin = _F_SP * m
    log = _MIN_LOG_HZ * np.exp(_LOGSTEP * (m - _MIN_LOG_MEL))
    return np.where(m >= _MIN_LOG_MEL, log, lin)


def mel_filters(sr=SAMPLE_RATE, n_fft=N_FFT, n_mels=N_MELS, fmin=0.0, fmax=None):
    """[n_mels, n_fft // 2 + 1] triangular filters, area-normalised."""
    fmax = sr / 2.0 if fmax is None else fmax
    bins = np.arange(n_fft // 2 + 1) * sr / n_fft                 # bin centre frequencies
    edges = mel_to_hz(np.linspace(hz_to_mel(fmin), hz_to_mel(fmax), n_mels + 2))
    w = np.zeros((n_mels, bins.size))
    for m in range(n_mels):
        lo, mid, hi = edges[m], edges[m + 1], edges[m + 2]
        up = (bins - lo) / (mid - lo)
        down = (hi - bins) / (hi - mid)
        w[m] = np.maximum(0.0, np.minimum(up, down)) * (2.0 / (hi - lo))
    return w


def hann(n=N_FFT):
    return 0.5 - 0.5 * np.cos(2.0 * np.pi * np.arange(n) / n)


def log_mel_frames(frames, filters=None):
    """[F, n_fft] sample frames -> [F, n_mels] log10 mel energies."""
    frames = np.asarray(frames, np.float64)
    n_fft = frames.shape[-1]
    filters = mel_filters(n_fft=n_fft) if filters is None else filters
    spec = np.fft.rfft(frames * hann(n_fft), axis=-1)
    energy = spec.real ** 2 + spec.imag ** 2
    return np.log10(np.maximum(energy @ filters.T, LOG_FLOOR))


def whole_signal(samples, n_fft=N_FFT, hop=HOP, filters=None):
    """Log-mel frames of a whole signal under the causal framing: the signal is
    preceded by n_fft - hop zeros and frame f covers padded samples
    [f*hop, f*hop + n_fft)."""
    x = np.concatenate([np.zeros(n_fft - hop), np.asarray(samples, np.float64)])
    count = (x.size - n_fft) // hop + 1
    frames = np.stack([x[f * hop:f * hop + n_fft] for f in range(count)])
    return log_mel_frames(frames, filters)


class RollingMel:
    """One stream's rolling sample buffer, fed step by step."""

    def __init__(self, n_fft=N_FFT, hop=HOP, filters=None):
        self.n_fft, self.hop = n_fft, hop
        self.filters = mel_filters(n_fft=n_fft) if filters is None else filters
        self.tail = np.zeros(n_fft - hop)          # the only samples a future frame can use

    def step(self, new_samples):
        """Append one step of samples; return the log-mel frames it completes."""
        new_samples = np.asarray(new_samples, np.float64)
        if new_samples.size % self.hop:
            raise ValueError("a step must carry whole hops")
        buf = np.concatenate([self.tail, new_samples])
        count = new_samples.size // self.hop
        frames = np.stack([buf[f * self.hop:f * self.hop + self.n_fft] for f in range(count)])
        self.tail = buf[buf.size - (self.n_fft - self.hop):].copy()
        return log_mel_frames(frames, self.filters)
