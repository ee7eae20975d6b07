"""Encoder chunk attention (F new frames per step against a rolling window of
cached frames) against the float64 oracle."""
import numpy as np
import pytest

from oracle import attention as att
from oracle import storage as stg
from rolling_window_kv_amd import synth

from gpu_util import check_close, device, f64, rkv_mod, run_encoder, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("H,d,F,W,extra", [(4, 64, 4, 30, 0), (3, 64, 4, 45, 5), (2, 128, 2, 37, 0),
                                           (5, 64, 8, 50, 3)])
def test_encoder_chunks_small(H, d, F, W, extra):
    rkv = rkv_mod()
    dev = device()
    L, S, T = 2, 3, 30
    cap = W + F + extra
    origins = np.array([0, 8, 400], np.int64)
    q, k, v = synth.encoder_pool(2005, L, S, T, F, H, d)
    cfg = rkv.make_cfg(S, L, num_q_heads=H, num_kv_heads=H, head_dim=d,
                       mode=rkv.RKV_MODE_ENC_CHUNK, new_rows=F)
    say(f"case: enc H={H} d={d} F={F} W={W} cap={cap}")
    _, out = run_encoder(rkv, cfg, cap, W, cap, origins, q.to(dev), k.to(dev), v.to(dev))
    got = f64(out)
    for l in range(L):
        for s in range(S):
            qh, kh, vh = (f64(x)[:, l, s] for x in (q, k, v))
            o = int(origins[s])
            exact = att.encoder_chunks(qh, kh, vh, W, 1e6, origin=o)
            check_close(got[:, l, s], np.stack([exact[t] for t in range(T)]), 2e-2,
                        f"enc l{l} s{s} vs exact")
            ring = stg.EncoderRing(H, d, W, F, 1e6, origin=o, cap=cap)
            sf = np.stack([ring.step(qh[t], kh[t], vh[t])[1] for t in range(T)])
            check_close(got[:, l, s], sf, 1e-3, f"enc l{l} s{s} vs storage-faithful",
                        ulp_slack=True)
