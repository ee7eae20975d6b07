"""Continuous-mode decoder restart (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring): plain Python integers,
one stream at a time.

voxtral.c rolling-KV explainer, section 四 (continuous mode for live
transcription): the runtime watches four conditions and restarts the decoder
when one holds.  The restart is hard -- no decoder context is carried over --
while the encoder cache and the streaming pipeline keep running.  The four
conditions, in the page's order:

  1. EOS: the model ends the current utterance;
  2. KV overflow: the decoder cache grows past STREAM_MAX_DECODE_KV (2000)
     positions; restarting bounds the attention cost;
  3. a run of non-text tokens: the decoder is looping on control tokens;
  4. a stall: audio advances but the decoder produces nothing (watchdog).

Readings taken where the page gives no detail:

  * one decoder position per clock step; the token of a step is a text token
    (id >= text_min), a control token (0 <= id < text_min), or none (id < 0);
  * the decoder length counts positions decoded since the last restart (the
    length of voxtral.c's decoder cache, which grows one row per token and is
    not compacted below 8192 positions); the overflow restart follows the step
    that brings it to max_kv, so no step attends over more than max_kv
    positions;
  * the non-text run counts consecutive control tokens (a text token or a
    step without a token ends it); the stall counts consecutive steps without
    a token;
  * the page gives no thresholds for 3 and 4: they are parameters (0 = off);
  * when several conditions hold at one step, the reason reported is the first
    in the page's order;
  * a restart clears the counters, and the stream's next step is the first of
    a fresh decoder context: its cache state is the initial state of a stream
    starting at the new origin (``restart_state``).
"""
from __future__ import annotations

from dataclasses import dataclass

from . import pages, schedule

NONE = 0
EOS = 1
KV_OVERFLOW = 2
NONTEXT_RUN = 3
STALL = 4


@dataclass
class RestartConfig:
    max_kv: int = pages.STREAM_MAX_DECODE_KV   # <= 0: off
    eos: int = -1                              # < 0: off
    text_min: int = 0                          # ids below this (and >= 0) are control tokens
    nontext_run: int = 0                       # <= 0: off
    stall: int = 0                             # <= 0: off


@dataclass
class Counters:
    decode_len: int = 0
    restarts: int = 0
    nontext: int = 0
    idle: int = 0


def policy_step(cfg: RestartConfig, c: Counters, token: int) -> int:
    """Account one clock step of one stream; return the restart reason (0: none)."""
    c.decode_len += 1
    is_control = 0 <= token < cfg.text_min
    c.nontext = c.nontext + 1 if is_control else 0
    c.idle = c.idle + 1 if token < 0 else 0
    if cfg.eos >= 0 and token == cfg.eos:
        reason = EOS
    elif cfg.max_kv > 0 and c.decode_len >= cfg.max_kv:
        reason = KV_OVERFLOW
    elif cfg.nontext_run > 0 and c.nontext >= cfg.nontext_run:
        reason = NONTEXT_RUN
    elif cfg.stall > 0 and c.idle >= cfg.stall:
        reason = STALL
    else:
        reason = NONE
    if reason != NONE:
        c.decode_len = 0
        c.nontext = 0
        c.idle = 0
        c.restarts += 1
    return reason


def policy_run(cfg: RestartConfig, tokens) -> list:
    """Reasons for a token sequence of one stream, from fresh counters."""
    c = Counters()
    return [policy_step(cfg, c, int(tok)) for tok in tokens]


def restart_state(mode: int, old: schedule.State, origin: int, dc: int = 1,
                  new_rows: int = 1) -> schedule.State:
    """Cache state of a stream restarted at ``origin``: a fresh stream there
    with the same window and capacity (no decoder context is kept)."""
    return schedule.init_state(mode, old.window, old.cap, origin, dc, new_rows)
