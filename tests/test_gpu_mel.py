"""The rolling log-mel front end on the GPU against the float64 oracle
(voxtral.c explainer, section 三: the mel buffer rolls): 12 steps for 5
streams of noise, tones and silence, at the 80 ms step (1280 samples, n_fft
400, hop 160) and with an odd 401-sample frame, compared frame by frame with
the oracle's rolling buffer; the carried tail bit-exact.

Both sides use the oracle's filterbank (oracle.mel.mel_filters rounded to
float32 on the host): the kernel gets it uploaded, the oracle the same
float32 values, so no device-built value feeds the oracle.  The library's
own filterbank (rkv_mel_filters_host) is checked against it separately."""
import numpy as np
import pytest
import torch

from oracle import mel

from gpu_util import device, rkv_mod, say

pytestmark = pytest.mark.gpu


def _audio(seed, S, T):
    rng = np.random.default_rng(seed)
    t = np.arange(T) / 16000.0
    x = np.zeros((S, T))
    x[0] = rng.standard_normal(T) * 0.1                                  # noise
    x[1] = 0.5 * np.sin(2 * np.pi * 440.0 * t) + 0.2 * np.sin(2 * np.pi * 3100.0 * t)
    x[2] = 0.0                                                           # silence
    x[3] = rng.standard_normal(T) * 1e-3 + 0.3 * np.sin(2 * np.pi * 7000.0 * t)
    x[4, T // 2:] = rng.standard_normal(T - T // 2)                      # silence, then loud
    return x.astype(np.float32)


@pytest.mark.parametrize("n_fft,hop,n_mels,per", [
    (400, 160, 128, 1280),      # the 80 ms step of 16 kHz audio
    (401, 100, 80, 800),        # odd frame: the two halves of each DFT sum differ in length
])
def test_rolling_mel_matches_oracle(n_fft, hop, n_mels, per):
    rkv = rkv_mod()
    dev = device()
    S, steps = 5, 12
    say(f"mel: n_fft={n_fft} hop={hop} n_mels={n_mels} samples/step={per}")
    cfg = rkv.make_mel_cfg(S, n_fft=n_fft, hop=hop, n_mels=n_mels, samples_per_step=per)
    filters32 = mel.mel_filters(sr=16000.0, n_fft=n_fft, n_mels=n_mels).astype(np.float32)
    # the library's filterbank is the oracle's, to within a float32 rounding
    lib_filters = rkv.rkv_mel_filters_host(cfg, 16000.0)
    ulp = np.spacing(np.abs(filters32)).astype(np.float32)
    assert np.all(np.abs(lib_filters - filters32) <= ulp), "rkv_mel_filters_host != oracle"
    fe = rkv.MelFrontend(cfg, device=dev, filters=filters32)
    assert np.array_equal(fe.filters.cpu().numpy(), filters32)
    x = _audio(5, S, steps * per)
    xd = torch.from_numpy(x).to(dev)
    out = torch.empty((steps, S, per // hop, n_mels), dtype=torch.float32, device=dev)
    for i in range(steps):
        fe.step(xd[:, i * per:(i + 1) * per].contiguous(), out[i])
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    filters = filters32.astype(np.float64)
    for s in range(S):
        roll = mel.RollingMel(n_fft=n_fft, hop=hop, filters=filters)  # the same float32 filterbank
        want = np.stack([roll.step(x[s, i * per:(i + 1) * per].astype(np.float64))
                         for i in range(steps)])
        eg, ew = 10.0 ** got[:, s], 10.0 ** want
        # float32 DFT sums of ~400 terms: energy error within 2e-5 of the
        # frame's largest band plus 1e-4 of the band itself
        tol = 2e-5 * ew.max(axis=-1, keepdims=True) + 1e-4 * ew
        err = np.abs(eg - ew)
        say(f"stream {s}: max energy error / tol {float((err / tol).max()):.3f}, "
            f"max |log10 diff| in bands above 1e-6 of the frame peak "
            f"{float(np.abs(got[:, s] - want)[ew > 1e-6 * ew.max(-1, keepdims=True)].max()):.2e}")
        assert np.all(err <= tol)
        tail = fe.tails[fe.parity][s].cpu().numpy()
        np.testing.assert_array_equal(tail, x[s, steps * per - (n_fft - hop):steps * per])
    assert np.all(got[:, 2] == np.float32(np.log10(np.float32(1e-10))))   # silence
