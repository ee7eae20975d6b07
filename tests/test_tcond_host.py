"""The library's host rule for the delay-token count (rkv_tcond_delay_tokens)
against the oracle, setting by setting, legal and illegal."""
import pytest

from oracle import tcond
from rolling_window_kv_amd import rkv


def test_delay_tokens_match_the_oracle():
    for clock in (40, 60, 80, 100, 120, 160, 200):
        for delay in range(-160, 2001, 20):
            try:
                want = tcond.delay_tokens(delay, clock)
            except ValueError:
                want = None
            if want is None:
                with pytest.raises(rkv.RkvError):
                    rkv.rkv_tcond_delay_tokens(delay, clock)
            else:
                assert rkv.rkv_tcond_delay_tokens(delay, clock) == want, (delay, clock)
