"""Per-step integer plans of the rolling KV cache (oracle).

Three modes, one state machine each, written in the order the pages give the
steps.  Every function works on one stream with plain Python integers.

REBASE (Audio8 explainer, "Rolling KV Cache 三步拆解", steps 1-2; model card,
"使用 vLLM 进行全天候推理": 30 s window with exact RoPE re-basing)
    A ring of W slots holds the last W tokens; when it is full the oldest token
    is pushed out by the new one.  Stored K carry positions relative to a base
    b.  Reading taken here where the pages are silent: one token is evicted per
    step (so attention always covers the last W positions) and the base moves
    in whole chunks of ``dc`` positions: b = dc * floor(o / dc) with o the
    oldest retained position; with dc = 1 the oldest retained K sits at
    relative position 0 ("re-zeroed into the window").  When b moves by D the
    retained K are rotated by R(-D) before the new K is written at p = t - b.

COMPACT (voxtral.c explainer, section 二: keep the newest window, move it to
slot 0, add the dropped count to kv_pos_offset; the rotary position of a row is
kv_pos_offset + physical index)
    A buffer of ``cap`` rows grows one row per step.  When it is full
    (len == cap, read from the garbled trigger as ``pos >= kv_cache_max`` and
    ``len >= window``), the oldest len - W rows are dropped, the newest W are
    moved to the front and kv_pos_offset grows by the number dropped; the new
    row then goes to physical index len.  K is never rewritten.

ENC (voxtral.c explainer, section 三: the encoder keeps a 750-position window
and encodes only new positions against cached K/V)
    Each step appends F frames at logical positions P..P+F-1 into a ring of
    ``cap`` >= W + F slots (slot = (position - origin) mod cap); frame j of the
    chunk attends to positions [max(origin, P - W), P + j].
"""
from __future__ import annotations

from dataclasses import dataclass, asdict

MODE_REBASE = 0
MODE_COMPACT = 1
MODE_ENC = 2


@dataclass
class Plan:
    """Integer plan of one step of one stream (field meanings by mode)."""
    t: int              # REBASE/COMPACT: step index of the new token; ENC: last new frame position
    pos: int            # rotary position of the first new row (relative to base, logical, logical)
    pos_offset: int     # REBASE: base b; COMPACT: kv_pos_offset; ENC: origin
    first_pos: int      # oldest position the new row(s) attend to (absolute/logical)
    evict_pos: int      # REBASE: position pushed out; COMPACT: first dropped; -1 none
    slot: int           # physical slot of the first new row
    n_valid: int        # rows valid after the append
    rebase_delta: int   # D: retained K rotate by R(-D) before the append (REBASE)
    compact_drop: int   # rows dropped by this step's compaction (COMPACT)
    evict_slot: int     # REBASE: slot of the pushed-out token; -1 none
    window: int
    cap: int
    new_rows: int

    def as_dict(self):
        return asdict(self)


@dataclass
class State:
    t: int
    origin: int
    pos_offset: int
    length: int
    window: int
    cap: int


def init_state(mode: int, window: int, cap: int, origin: int = 0, dc: int = 1,
               new_rows: int = 1) -> State:
    """State before the first step of a stream whose first position is ``origin``."""
    if mode == MODE_REBASE:
        if cap != window:
            raise ValueError("the re-base ring has exactly W slots")
        return State(origin - 1, origin, dc * (origin // dc), 0, window, cap)
    if mode == MODE_COMPACT:
        if cap <= window:
            raise ValueError("compaction needs room beyond the window")
        return State(origin - 1, origin, origin, 0, window, cap)
    if mode == MODE_ENC:
        if cap < window + new_rows:
            raise ValueError("the encoder ring needs W + F slots")
        return State(origin - 1, origin, origin, 0, window, cap)
    raise ValueError(mode)


def step(mode: int, st: State, dc: int = 1, new_rows: int = 1) -> Plan:
    """Advance ``st`` by one step in place and return the step's plan."""
    if mode == MODE_REBASE:
        st.t += 1
        if st.length == st.window:          # full: the oldest token leaves
            evict_pos = st.t - st.window
            evict_slot = (st.t - st.origin) % st.window
        else:
            st.length += 1
            evict_pos = -1
            evict_slot = -1
        slot = (st.t - st.origin) % st.window
        oldest = st.t - st.length + 1
        new_base = dc * (oldest // dc)
        delta = new_base - st.pos_offset
        st.pos_offset = new_base
        return Plan(st.t, st.t - new_base, new_base, oldest, evict_pos, slot,
                    st.length, delta, 0, evict_slot, st.window, st.cap, 1)
    if mode == MODE_COMPACT:
        st.t += 1
        drop = 0
        evict_pos = -1
        if st.length >= st.cap and st.length >= st.window:
            drop = st.length - st.window
            evict_pos = st.pos_offset
            st.pos_offset += drop
            st.length = st.window
        slot = st.length
        st.length += 1
        return Plan(st.t, st.pos_offset + slot, st.pos_offset, st.pos_offset,
                    evict_pos, slot, st.length, 0, drop, -1, st.window, st.cap, 1)
    if mode == MODE_ENC:
        first_new = st.t + 1
        st.t += new_rows
        slot = (first_new - st.origin) % st.cap
        st.length = min(st.length + new_rows, st.cap)
        first_pos = max(st.origin, first_new - st.window)
        return Plan(st.t, first_new, st.origin, first_pos, -1, slot, st.length,
                    0, 0, -1, st.window, st.cap, new_rows)
    raise ValueError(mode)


def run(mode: int, steps: int, window: int, cap: int, origin: int = 0,
        dc: int = 1, new_rows: int = 1):
    """Plans of ``steps`` consecutive steps of a fresh stream."""
    st = init_state(mode, window, cap, origin, dc, new_rows)
    return [step(mode, st, dc, new_rows) for _ in range(steps)]


def enc_slot_positions(plan: Plan, origin: int):
    """Logical position held by each valid slot of the encoder ring after ``plan``.

    Returns a list indexed by slot (None for slots not yet written).
    """
    last = plan.t
    out = [None] * plan.cap
    for r in range(plan.cap):
        # newest position p <= last with (p - origin) % cap == r
        back = ((last - origin) - r) % plan.cap
        p = last - back
        out[r] = p if p >= origin else None
    return out
