"""Pins for oracle.restart (voxtral.c explainer, section 四: continuous-mode
decoder restart).  Each expectation is written out by hand from the rule it
tests -- positions of restarts in short synthetic token sequences, and the
closed form of the overflow period -- not recomputed with the oracle's code."""
import pytest

from oracle import pages
from oracle import restart as rs
from oracle import schedule as sch

TEXT = 100      # a text token (text ids start at 10 below)
CTRL = 3        # a control token
NONE = -1       # no token this step


def restarts_at(reasons):
    return [i for i, r in enumerate(reasons) if r != rs.NONE]


def test_overflow_period_is_the_page_limit():
    # all text: a fresh context every 2000 positions; restart after steps
    # 1999, 3999, 5999 (0-based), so every context holds exactly 2000 positions
    cfg = rs.RestartConfig(max_kv=pages.STREAM_MAX_DECODE_KV, text_min=10)
    reasons = rs.policy_run(cfg, [TEXT] * 6500)
    assert restarts_at(reasons) == [1999, 3999, 5999]
    assert all(reasons[i] == rs.KV_OVERFLOW for i in (1999, 3999, 5999))


def test_overflow_small_limit():
    cfg = rs.RestartConfig(max_kv=3, text_min=10)
    assert restarts_at(rs.policy_run(cfg, [TEXT] * 10)) == [2, 5, 8]


def test_eos_restarts_where_it_appears_and_starts_a_new_context():
    cfg = rs.RestartConfig(max_kv=5, eos=7, text_min=10)
    toks = [TEXT, 7, TEXT, TEXT, TEXT, TEXT, TEXT, 7, 7, TEXT]
    # EOS at 1, 7, 8; after the EOS at 1 the context restarts, so the
    # overflow of 5 positions comes at 6 (positions 2..6), not at 4
    reasons = rs.policy_run(cfg, toks)
    assert restarts_at(reasons) == [1, 6, 7, 8]
    assert [reasons[i] for i in (1, 6, 7, 8)] == [rs.EOS, rs.KV_OVERFLOW, rs.EOS, rs.EOS]


def test_nontext_run():
    cfg = rs.RestartConfig(max_kv=0, text_min=10, nontext_run=3)
    # runs of control tokens of length 2, 3 and 7, separated by text
    toks = [CTRL, CTRL, TEXT, CTRL, CTRL, CTRL, TEXT] + [CTRL] * 7 + [TEXT]
    # run 2 (indices 3..5) restarts at its 3rd token (5); run 3 (7..13)
    # restarts at its 3rd and 6th tokens (9, 12): the count starts over
    reasons = rs.policy_run(cfg, toks)
    assert restarts_at(reasons) == [5, 9, 12]
    assert all(reasons[i] == rs.NONTEXT_RUN for i in (5, 9, 12))


def test_stall_counts_steps_without_a_token():
    cfg = rs.RestartConfig(max_kv=0, text_min=10, stall=4)
    toks = [NONE] * 3 + [CTRL] + [NONE] * 9 + [TEXT]
    # the control token at 3 ends the first idle run (3 steps); the next run
    # (4..12) restarts at its 4th and 8th steps (7, 11)
    reasons = rs.policy_run(cfg, toks)
    assert restarts_at(reasons) == [7, 11]
    assert all(reasons[i] == rs.STALL for i in (7, 11))


def test_text_ends_a_nontext_run_and_a_token_ends_a_stall():
    cfg = rs.RestartConfig(max_kv=0, text_min=10, nontext_run=2, stall=2)
    toks = [CTRL, TEXT, CTRL, NONE, CTRL, NONE, TEXT, NONE]
    assert restarts_at(rs.policy_run(cfg, toks)) == []


def test_reason_order_follows_the_page():
    # EOS and overflow at the same step: EOS
    cfg = rs.RestartConfig(max_kv=2, eos=5, text_min=10)
    assert rs.policy_run(cfg, [TEXT, 5]) == [rs.NONE, rs.EOS]
    # overflow and a non-text run at the same step: overflow
    cfg = rs.RestartConfig(max_kv=2, text_min=10, nontext_run=2)
    assert rs.policy_run(cfg, [CTRL, CTRL]) == [rs.NONE, rs.KV_OVERFLOW]
    # a control-token EOS id with a non-text run: EOS
    cfg = rs.RestartConfig(max_kv=0, eos=CTRL, text_min=10, nontext_run=1)
    assert rs.policy_run(cfg, [CTRL]) == [rs.EOS]
    # a non-text run and a stall cannot coincide; the stall alone:
    cfg = rs.RestartConfig(max_kv=0, text_min=10, nontext_run=1, stall=1)
    assert rs.policy_run(cfg, [NONE, CTRL]) == [rs.STALL, rs.NONTEXT_RUN]


def test_everything_off_never_restarts():
    cfg = rs.RestartConfig(max_kv=0, eos=-1, text_min=10, nontext_run=0, stall=0)
    toks = [CTRL] * 50 + [NONE] * 50 + [TEXT] * 50
    assert restarts_at(rs.policy_run(cfg, toks)) == []


@pytest.mark.parametrize("mode,W,cap,dc,F", [(sch.MODE_REBASE, 7, 7, 3, 1),
                                             (sch.MODE_COMPACT, 5, 8, 1, 1),
                                             (sch.MODE_ENC, 6, 9, 1, 2)])
def test_restarted_stream_is_a_fresh_stream(mode, W, cap, dc, F):
    # a stream that ran 23 steps from 4 and restarts at 100 plans exactly like
    # a stream that starts at 100 (brute force: two runs compared)
    st = sch.init_state(mode, W, cap, 4, dc, F)
    for _ in range(23):
        sch.step(mode, st, dc, F)
    st = rs.restart_state(mode, st, 100, dc, F)
    fresh = sch.init_state(mode, W, cap, 100, dc, F)
    a = [sch.step(mode, st, dc, F).as_dict() for _ in range(3 * cap)]
    b = [sch.step(mode, fresh, dc, F).as_dict() for _ in range(3 * cap)]
    assert a == b
    assert a[0]["n_valid"] == F and a[0]["t"] == 100 + F - 1
