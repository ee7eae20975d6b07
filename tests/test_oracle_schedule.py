"""Pins for oracle.schedule: brute-force simulations of the ring, the
compaction buffer (a Python list sliced like the memmove) and the encoder
ring, plus closed forms for the workloads' re-base and compaction counts."""
from collections import deque

import pytest

from oracle import schedule as sch


@pytest.mark.parametrize("W,dc,origin", [(5, 1, 0), (5, 2, 0), (7, 3, 11), (375, 25, 0), (188, 25, 4321)])
def test_rebase_ring_against_brute_force(W, dc, origin):
    plans = sch.run(sch.MODE_REBASE, 3 * W + 2 * dc + 5, W, W, origin, dc)
    ring = deque()                  # (position, slot), oldest first
    base = None
    for i, p in enumerate(plans):
        t = origin + i
        if len(ring) == W:
            old_pos, slot = ring.popleft()
            assert p.evict_pos == old_pos and p.evict_slot == slot
        else:
            slot = len(ring)
            assert p.evict_pos == -1 and p.evict_slot == -1
        ring.append((t, slot))
        assert p.t == t and p.slot == slot and p.n_valid == len(ring)
        oldest = ring[0][0]
        assert p.first_pos == oldest
        # base: the largest multiple of dc not above the oldest retained position
        b = max(m for m in range(0, oldest + 1) if m % dc == 0)
        assert p.pos_offset == b
        assert p.rebase_delta == (0 if base is None else b - base)
        base = b
        assert p.pos == t - b
        rel = sorted(pos - b for pos, _ in ring)
        assert 0 <= rel[0] and rel[-1] <= W + dc - 2
        if dc == 1 and len(ring) == W:
            assert rel == list(range(W))          # oldest retained re-zeroed at 0


def test_rebase_counts_for_the_chunked_workload():
    # W = 375, chunks of 25: the first re-base when the oldest retained reaches 25.
    plans = sch.run(sch.MODE_REBASE, 10000, 375, 375, 0, 25)
    steps = [p.t for p in plans if p.rebase_delta]
    assert steps[0] == 399 and steps[1] == 424
    assert len(steps) == (9999 - 399) // 25 + 1
    assert all(p.rebase_delta in (0, 25) for p in plans)
    every = sch.run(sch.MODE_REBASE, 1000, 375, 375, 0, 1)
    assert [p.t for p in every if p.rebase_delta] == list(range(375, 1000))


@pytest.mark.parametrize("W,cap,origin", [(3, 5, 0), (4, 4 + 1, 9), (8192, 9216, 0)])
def test_compaction_against_list_simulation(W, cap, origin):
    steps = 4 * cap if cap < 100 else 20000
    plans = sch.run(sch.MODE_COMPACT, steps, W, cap, origin)
    buf = []                        # logical positions, physical index = list index
    offset = origin
    n_compactions = 0
    for i, p in enumerate(plans):
        t = origin + i
        drop = 0
        if len(buf) == cap:
            drop = len(buf) - W
            buf = buf[drop:]        # the memmove of the newest W rows to slot 0
            offset += drop
            n_compactions += 1
        assert p.compact_drop == drop
        buf.append(t)
        assert p.slot == len(buf) - 1 and p.n_valid == len(buf) and p.pos_offset == offset
        assert p.pos == t               # offset + physical index is the true position
        if cap < 100:
            assert all(offset + j == pos for j, pos in enumerate(buf))
        assert len(buf) <= cap
    if (W, cap) == (8192, 9216):
        # first compaction when the buffer is full at step 9216, then every 1024 steps
        assert n_compactions == (19999 - 9216) // 1024 + 1 == 11


@pytest.mark.parametrize("W,F,cap,origin", [(7, 4, 11, 0), (7, 4, 13, 3), (750, 4, 754, 0)])
def test_encoder_ring_against_brute_force(W, F, cap, origin):
    n_steps = 3 * cap // F + 3
    plans = sch.run(sch.MODE_ENC, n_steps, W, cap, origin, 1, F)
    slots = {}
    for n, p in enumerate(plans):
        P = origin + n * F
        assert p.pos == P and p.t == P + F - 1 and p.slot == (P - origin) % cap
        for j in range(F):
            slots[(P + j - origin) % cap] = P + j
        assert p.n_valid == min((n + 1) * F, cap)
        got = sch.enc_slot_positions(p, origin)
        for r in range(cap):
            assert got[r] == slots.get(r)
        # every position a row of this chunk may attend to is still in the ring
        held = {pos for pos in slots.values()}
        assert p.first_pos == max(origin, P - W)
        for pos in range(p.first_pos, P + F):
            assert pos in held


def test_init_validation():
    with pytest.raises(ValueError):
        sch.init_state(sch.MODE_REBASE, 5, 6)
    with pytest.raises(ValueError):
        sch.init_state(sch.MODE_COMPACT, 5, 5)
    with pytest.raises(ValueError):
        sch.init_state(sch.MODE_ENC, 750, 753, new_rows=4)
