"""Pins for oracle.pages against the constants the pages print
(tests/golden/page_constants.json, each entry with its page and section)."""
import json
import os

import pytest

from oracle import pages

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def test_window_positions_per_clock():
    for clock, w in GOLDEN["window_positions"]["value"].items():
        assert pages.window_positions(int(clock)) == w
    assert pages.WINDOW_SECONDS == GOLDEN["window_seconds"]["value"]


def test_clock_table():
    for row in GOLDEN["clocks"]["value"]:
        assert pages.frame_len(row["clock_ms"]) == row["frame_len"]
        # the pages print 8.3 for 1000/120
        assert round(pages.decisions_per_second(row["clock_ms"]), 2 if row["clock_ms"] != 120 else 1) == row["decisions_per_s"]
    assert pages.TOWER_FRAME_MS == GOLDEN["tower_frame_ms"]["value"]


def test_samples_and_delay_tokens():
    assert pages.samples_per_step(80) == GOLDEN["samples_per_step_80ms"]["value"]
    assert pages.num_delay_tokens(480, 80) == GOLDEN["num_delay_tokens_480ms_80ms"]["value"]
    with pytest.raises(ValueError):
        pages.num_delay_tokens(500, 80)


def test_model_geometry():
    dec = GOLDEN["decoder"]["value"]
    assert (pages.DECODER_LAYERS, pages.DECODER_HIDDEN, pages.DECODER_Q_HEADS,
            pages.DECODER_KV_HEADS) == (dec["layers"], dec["hidden"], dec["q_heads"], dec["kv_heads"])
    assert pages.head_dim(pages.DECODER_HIDDEN, pages.DECODER_Q_HEADS) == dec["head_dim"]
    enc = GOLDEN["encoder"]["value"]
    assert (pages.ENCODER_LAYERS, pages.ENCODER_HIDDEN, pages.ENCODER_WINDOW) == (enc["layers"], enc["hidden"], enc["window"])
    vox = GOLDEN["voxtral"]["value"]
    assert pages.VOX_DEC_WINDOW == vox["VOX_DEC_WINDOW"]
    assert pages.VOX_ENC_WINDOW == vox["VOX_ENC_WINDOW"]
    assert pages.STREAM_MAX_DECODE_KV == vox["STREAM_MAX_DECODE_KV"]
