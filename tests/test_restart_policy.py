"""The library's continuous-mode restart policy (rkv_restart_step, host code
of librkv.so) against the oracle's reading of the voxtral.c explainer,
section 四: the same restart steps and reasons, decision by decision, on
seeded synthetic token streams that exercise every trigger; plus argument
checks.  No GPU is involved."""
import ctypes

import numpy as np
import pytest

from oracle import restart as rs

CASES = [
    # max_kv, eos, text_min, nontext_run, stall, token mix (text, control, none, eos)
    (2000, -1, 10, 0, 0, (1.0, 0.0, 0.0, 0.0)),
    (50, 7, 10, 5, 6, (0.6, 0.25, 0.14, 0.01)),
    (0, 3, 10, 3, 0, (0.5, 0.45, 0.04, 0.01)),
    (0, -1, 10, 0, 4, (0.3, 0.0, 0.7, 0.0)),
    (30, 0, 1, 2, 2, (0.4, 0.3, 0.3, 0.0)),
]


@pytest.fixture(scope="module")
def rkv():
    from rolling_window_kv_amd import rkv as mod
    mod.lib()
    return mod


def _tokens(seed, S, T, text_min, eos, mix):
    rng = np.random.default_rng(seed)
    kind = rng.choice(4, size=(T, S), p=np.asarray(mix) / sum(mix))
    text = rng.integers(max(text_min, 10), 50000, size=(T, S))
    ctrl = rng.integers(0, max(text_min, 1), size=(T, S)) if text_min > 0 else text
    tok = np.where(kind == 0, text, np.where(kind == 1, ctrl, -1))
    if eos >= 0:
        tok = np.where(kind == 3, eos, tok)
    return tok.astype(np.int32)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_policy_matches_oracle(rkv, case):
    max_kv, eos, text_min, run, stall, mix = CASES[case]
    S, T = 37, 4500
    tok = _tokens(100 + case, S, T, text_min, eos, mix)
    cfg = rkv.make_restart_cfg(max_kv, eos, text_min, run, stall)
    ocfg = rs.RestartConfig(max_kv, eos, text_min, run, stall)
    state = np.zeros(S, rkv.RESTART_STATE_DTYPE)
    counters = [rs.Counters() for _ in range(S)]
    total = 0
    for t in range(T):
        restart, reason = rkv.rkv_restart_step(cfg, state, tok[t])
        want = np.array([rs.policy_step(ocfg, counters[s], int(tok[t, s])) for s in range(S)])
        assert np.array_equal(reason, want), f"step {t}"
        assert np.array_equal(restart, np.flatnonzero(want)), f"step {t}"
        total += restart.size
    assert np.array_equal(state["decode_len"], [c.decode_len for c in counters])
    assert np.array_equal(state["restarts"], [c.restarts for c in counters])
    assert np.array_equal(state["nontext"], [c.nontext for c in counters])
    assert np.array_equal(state["idle"], [c.idle for c in counters])
    assert total > 0


def test_policy_rejects_bad_arguments(rkv):
    cfg = rkv.make_restart_cfg()
    st = np.zeros(4, rkv.RESTART_STATE_DTYPE)
    tok = np.zeros(4, np.int32)
    f = rkv.lib().rkv_restart_step
    assert f(None, st.ctypes.data, 4, tok.ctypes.data, None, None) == rkv.RKV_EINVAL
    assert f(ctypes.byref(cfg), None, 4, tok.ctypes.data, None, None) == rkv.RKV_EINVAL
    assert f(ctypes.byref(cfg), st.ctypes.data, 4, None, None, None) == rkv.RKV_EINVAL
    assert f(ctypes.byref(cfg), st.ctypes.data, 0, tok.ctypes.data, None, None) == rkv.RKV_EINVAL
    bad = rkv.make_restart_cfg(text_token_min=-1)
    assert f(ctypes.byref(bad), st.ctypes.data, 4, tok.ctypes.data, None, None) == rkv.RKV_EINVAL
    # outputs are optional
    assert f(ctypes.byref(cfg), st.ctypes.data, 4, tok.ctypes.data, None, None) == 0
    assert np.all(st["decode_len"] == 1)
