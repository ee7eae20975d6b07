"""rkv_state_advance_host (host code of librkv.so, no GPU): advancing stream
states by N steps on the host must give the states that N steps of the
oracle's schedule give (oracle/schedule.py, itself pinned by
test_oracle_schedule.py), in every mode, across re-base chunk boundaries,
compactions and encoder-ring wrap-around; invalid states and arguments are
rejected without changing anything."""
import numpy as np
import pytest

from oracle import schedule as sch

from rolling_window_kv_amd import rkv


def _oracle_states(mode, windows, caps, origins, dc, F, steps):
    out = []
    for W, cap, o in zip(windows, caps, origins):
        st = sch.init_state(mode, int(W), int(cap), int(o), dc, F)
        for _ in range(steps):
            sch.step(mode, st, dc, F)
        out.append((st.t, st.origin, st.pos_offset, st.length, st.window, st.cap))
    return out


CASES = [
    # name, mode, windows, caps (None: = windows), origins, dc, F, step counts
    ("rebase-dc25", rkv.RKV_MODE_REBASE, [375, 375, 100], None, [0, 7, 1234], 25, 1,
     [0, 1, 99, 100, 374, 375, 376, 399, 400, 1000]),
    ("rebase-dc1", rkv.RKV_MODE_REBASE, [64, 3], None, [0, 5], 1, 1, [0, 2, 63, 64, 65, 500]),
    ("compact", rkv.RKV_MODE_COMPACT, [8192, 64, 10], [9216, 80, 11], [0, 3, 100], 1, 1,
     [0, 9, 10, 11, 12, 80, 81, 97, 9216, 9217, 20000]),
    ("encoder", rkv.RKV_MODE_ENC_CHUNK, [750, 60], [754, 64], [0, 17], 1, 4,
     [0, 1, 15, 16, 17, 188, 189, 190, 500]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_host_advance_matches_oracle_schedule(case):
    name, mode, windows, caps, origins, dc, F, counts = case
    caps = windows if caps is None else caps
    S = len(windows)
    cfg = rkv.make_cfg(S, 1, num_q_heads=(4 if mode == rkv.RKV_MODE_ENC_CHUNK else 16),
                       num_kv_heads=(4 if mode == rkv.RKV_MODE_ENC_CHUNK else 2),
                       head_dim=(64 if mode == rkv.RKV_MODE_ENC_CHUNK else 128), mode=mode,
                       rebase_chunk=dc, new_rows=F, max_cap=max(caps))
    w = np.array(windows, np.int32)
    c = np.array(caps, np.int32)
    o = np.array(origins, np.int64)
    for n in counts:
        st = rkv.rkv_state_init_host(cfg, w, c, o)
        rkv.rkv_state_advance_host(cfg, st, n)
        want = _oracle_states(mode, windows, caps, origins, dc, F, n)
        got = [(int(x["t"]), int(x["origin"]), int(x["pos_offset"]), int(x["len"]),
                int(x["window"]), int(x["cap"])) for x in st]
        assert got == want, (name, n)
    # advancing in two parts equals advancing at once
    a = rkv.rkv_state_init_host(cfg, w, c, o)
    b = rkv.rkv_state_init_host(cfg, w, c, o)
    rkv.rkv_state_advance_host(cfg, a, 37)
    rkv.rkv_state_advance_host(cfg, a, 400)
    rkv.rkv_state_advance_host(cfg, b, 437)
    assert a.tobytes() == b.tobytes()


def test_host_advance_rejects_bad_input():
    cfg = rkv.make_cfg(2, 1, mode=rkv.RKV_MODE_COMPACT, max_cap=80)
    st = rkv.rkv_state_init_host(cfg, np.array([64, 64], np.int32), np.array([80, 80], np.int32),
                                 np.array([0, 0], np.int64))
    with pytest.raises(rkv.RkvError) as e:
        rkv.rkv_state_advance_host(cfg, st, -1)
    assert e.value.status == rkv.RKV_EINVAL
    bad = st.copy()
    bad[1]["len"] = 81               # more rows than the capacity
    keep = bad.copy()
    with pytest.raises(rkv.RkvError) as e:
        rkv.rkv_state_advance_host(cfg, bad, 5)
    assert e.value.status == rkv.RKV_ESTATE
    assert bad.tobytes() == keep.tobytes()      # nothing changed
    bad = st.copy()
    bad[0]["cap"] = 64               # compaction needs room beyond the window
    with pytest.raises(rkv.RkvError) as e:
        rkv.rkv_state_advance_host(cfg, bad, 5)
    assert e.value.status == rkv.RKV_ESTATE
    bad = st.copy()
    bad[0]["cap"] = 96               # beyond max_cap
    with pytest.raises(rkv.RkvError) as e:
        rkv.rkv_state_advance_host(cfg, bad, 5)
    assert e.value.status == rkv.RKV_ESTATE
    with pytest.raises(ValueError):
        rkv.rkv_state_advance_host(cfg, st[:1].copy(), 5)
