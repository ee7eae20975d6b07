"""Constants the pages state, and the sizes derived from them (oracle).

Each helper turns a stated relation into a number the workloads use; the
values are pinned against ``tests/golden/page_constants.json``.
"""
from __future__ import annotations

import math

# Audio8 explainer "模型一览" and model card "架构": 30 s native context.
WINDOW_SECONDS = 30.0
# Audio8 explainer "三档音频时钟": the audio tower's base frame is 20 ms.
TOWER_FRAME_MS = 20
# Model card "使用" (usage snippet): 16 kHz input audio.
SAMPLE_RATE = 16000
# Model card "架构" checkpoint specification.
DECODER_LAYERS = 36
DECODER_HIDDEN = 2048
DECODER_Q_HEADS = 16
DECODER_KV_HEADS = 2
ENCODER_LAYERS = 32
ENCODER_HIDDEN = 1280
ENCODER_WINDOW = 750
# voxtral.c explainer, section 一 window table and section 四.
VOX_DEC_WINDOW = 8192
VOX_ENC_WINDOW = 750
STREAM_MAX_DECODE_KV = 2000


def window_positions(clock_ms: float, window_s: float = WINDOW_SECONDS) -> int:
    """Decoder window in clock steps: 30 s of audio over the clock period.

    30 s / 160 ms is 187.5; a window must hold whole steps, and the half step
    is rounded up so the window covers at least 30 s (188).
    """
    return int(math.ceil(window_s * 1000.0 / clock_ms - 1e-9))


def frame_len(clock_ms: int) -> int:
    """Tower frames packed per clock step (20 ms frames)."""
    if clock_ms % TOWER_FRAME_MS:
        raise ValueError("the clock must be a whole number of 20 ms frames")
    return clock_ms // TOWER_FRAME_MS


def decisions_per_second(clock_ms: float) -> float:
    """One text token per clock step."""
    return 1000.0 / clock_ms


def samples_per_step(clock_ms: int, sample_rate: int = SAMPLE_RATE) -> int:
    return sample_rate * clock_ms // 1000


def num_delay_tokens(target_delay_ms: int, clock_ms: int) -> int:
    """Delay in clock steps; the delay must be a whole number of clocks."""
    if target_delay_ms % clock_ms:
        raise ValueError("target_delay_ms must be an integer multiple of the clock")
    return target_delay_ms // clock_ms


def head_dim(hidden: int, heads: int) -> int:
    if hidden % heads:
        raise ValueError("hidden size must split evenly over the heads")
    return hidden // heads
