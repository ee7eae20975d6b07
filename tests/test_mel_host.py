"""Host side of the rolling log-mel front end (no GPU): the library's
filterbank against the oracle's, and argument checks of rkv_mel_step that
fail before any HIP call."""
import ctypes

import numpy as np
import pytest

from oracle import mel


@pytest.fixture(scope="module")
def rkv():
    from rolling_window_kv_amd import rkv as mod
    mod.lib()
    return mod


@pytest.mark.parametrize("n_fft,n_mels,sr", [(400, 128, 16000.0), (512, 80, 22050.0)])
def test_filterbank_matches_oracle(rkv, n_fft, n_mels, sr):
    cfg = rkv.make_mel_cfg(2, n_fft=n_fft, n_mels=n_mels)
    got = rkv.rkv_mel_filters_host(cfg, sr).astype(np.float64)
    want = mel.mel_filters(sr=sr, n_fft=n_fft, n_mels=n_mels)
    np.testing.assert_allclose(got, want, rtol=2.0 ** -23, atol=1e-12)


def test_mel_step_rejects_bad_arguments(rkv):
    F = ctypes.c_void_p(0x10000)
    G = ctypes.c_void_p(0x20000)
    N = None
    f = rkv.lib().rkv_mel_step
    ok = rkv.make_mel_cfg(4)
    c = ctypes.byref(ok)
    assert f(N, F, G, F, F, F, N) == rkv.RKV_EINVAL
    assert f(c, N, G, F, F, F, N) == rkv.RKV_EINVAL
    assert f(c, F, G, F, N, F, N) == rkv.RKV_EINVAL
    # tails overlap: 4 streams x 240 floats from 0x10000
    assert f(c, F, ctypes.c_void_p(0x10000 + 4 * 240 * 4 - 4), F, F, F, N) == rkv.RKV_EINVAL
    assert f(c, F, G, ctypes.c_void_p(0x30002), F, F, N) == rkv.RKV_EALIGN
    for bad in (rkv.make_mel_cfg(4, samples_per_step=1000),      # not whole hops
                rkv.make_mel_cfg(4, samples_per_step=160),       # shorter than the tail
                rkv.make_mel_cfg(4, n_fft=1024),                 # window too long
                rkv.make_mel_cfg(4, hop=500),                    # hop beyond the window
                rkv.make_mel_cfg(0)):
        assert f(ctypes.byref(bad), F, G, F, F, F, N) == rkv.RKV_EINVAL
    assert rkv.lib().rkv_mel_filters_host(c, 0.0, F) == rkv.RKV_EINVAL
    assert rkv.rkv_last_hip_error() == 0
