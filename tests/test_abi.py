"""C ABI checks that need no GPU: the library loads, exports every entry point
include/rkv.h declares, struct layouts agree with the binding, and host-side
validation rejects bad arguments before any HIP call (fake pointers used here
always fail validation, so nothing is ever launched)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import schedule as sch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rkv.h")


@pytest.fixture(scope="module")
def rkv():
    from rolling_window_kv_amd import rkv as mod
    if not os.path.exists(mod.lib_path()):
        from rolling_window_kv_amd import build
        build.build()
    mod.lib()
    return mod


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(rkv_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_entry_points(rkv):
    assert declared_functions() == sorted(rkv.ENTRY_POINTS)


def test_library_exports_every_declared_symbol(rkv):
    out = subprocess.run(["nm", "-D", "--defined-only", rkv.lib_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(rkv.lib(), name) is not None


def test_struct_sizes(rkv):
    assert ctypes.sizeof(rkv.rkv_cfg) == 56
    assert ctypes.sizeof(rkv.rkv_kv_view) == 64
    assert rkv.STATE_DTYPE.itemsize == 48
    assert rkv.PLAN_DTYPE.itemsize == 9344
    assert ctypes.sizeof(rkv.rkv_restart_cfg) == 24
    assert rkv.RESTART_STATE_DTYPE.itemsize == 24


def test_version_and_strerror(rkv):
    assert rkv.rkv_version() == 1
    for code in (0, -1, -2, -3, -4, -5, -6, -99):
        assert isinstance(rkv.strerror(code), str) and rkv.strerror(code)
    assert rkv.rkv_last_hip_error() == 0


def good_cfg(rkv, **kw):
    base = dict(num_streams=4, num_layers=2, num_q_heads=16, num_kv_heads=2, head_dim=128,
                mode=rkv.RKV_MODE_REBASE, rebase_chunk=25, max_cap=375)
    base.update(kw)
    return rkv.make_cfg(**base)


def test_cfg_validation(rkv):
    assert rkv.rkv_validate_cfg(good_cfg(rkv)) == 0
    bad = [
        (dict(num_streams=0), rkv.RKV_EINVAL),
        (dict(head_dim=96), rkv.RKV_EUNSUPPORTED),
        (dict(num_q_heads=15), rkv.RKV_EINVAL),
        (dict(num_q_heads=32, num_kv_heads=2), rkv.RKV_EUNSUPPORTED),
        (dict(rebase_chunk=0), rkv.RKV_EINVAL),
        (dict(mode=7), rkv.RKV_EUNSUPPORTED),
        (dict(flags=16), rkv.RKV_EUNSUPPORTED),
        (dict(rope_base=-1.0), rkv.RKV_EINVAL),
        (dict(rope_base=float("inf")), rkv.RKV_EINVAL),
        (dict(softmax_scale=-1.0), rkv.RKV_EINVAL),
        (dict(new_rows=2), rkv.RKV_EINVAL),
        (dict(mode=rkv.RKV_MODE_COMPACT, flags=rkv.RKV_F_COMPENSATED), rkv.RKV_EUNSUPPORTED),
        (dict(mode=rkv.RKV_MODE_ENC_CHUNK, new_rows=4), rkv.RKV_EINVAL),       # Hq != Hkv
        (dict(mode=rkv.RKV_MODE_ENC_CHUNK, num_q_heads=20, num_kv_heads=20, head_dim=64,
              new_rows=9), rkv.RKV_EUNSUPPORTED),
    ]
    for kw, code in bad:
        assert rkv.rkv_validate_cfg(good_cfg(rkv, **kw)) == code, kw
    enc = good_cfg(rkv, mode=rkv.RKV_MODE_ENC_CHUNK, num_q_heads=20, num_kv_heads=20,
                   head_dim=64, new_rows=4)
    assert rkv.rkv_validate_cfg(enc) == 0


@pytest.mark.parametrize("mode,W,cap,dc,F", [(0, 375, 375, 25, 1), (0, 188, 188, 1, 1),
                                              (1, 8192, 9216, 1, 1), (2, 750, 754, 1, 4)])
def test_state_init_matches_oracle(rkv, mode, W, cap, dc, F):
    kw = dict(mode=mode, rebase_chunk=dc, new_rows=F)
    if mode == 2:
        kw.update(num_q_heads=20, num_kv_heads=20, head_dim=64)
    cfg = good_cfg(rkv, max_cap=cap, **kw)
    origins = np.array([0, 1, 4321, 5000], np.int64)
    st = rkv.rkv_state_init_host(cfg, W, cap, origins)
    for s in range(4):
        ref = sch.init_state(mode, W, cap, int(origins[s]), dc, F)
        assert (st["t"][s], st["origin"][s], st["pos_offset"][s], st["len"][s],
                st["window"][s], st["cap"][s]) == (ref.t, ref.origin, ref.pos_offset,
                                                    ref.length, ref.window, ref.cap)


def test_state_init_rejects_inconsistent_streams(rkv):
    cfg = good_cfg(rkv)
    with pytest.raises(rkv.RkvError) as e:
        rkv.rkv_state_init_host(cfg, 375, 376, 0)
    assert e.value.status == rkv.RKV_ESTATE
    with pytest.raises(rkv.RkvError):
        rkv.rkv_state_init_host(cfg, 375, 375, -1)
    ccfg = good_cfg(rkv, mode=rkv.RKV_MODE_COMPACT, max_cap=9216)
    with pytest.raises(rkv.RkvError):
        rkv.rkv_state_init_host(ccfg, 8192, 8192, 0)
    ecfg = good_cfg(rkv, mode=rkv.RKV_MODE_ENC_CHUNK, num_q_heads=20, num_kv_heads=20,
                    head_dim=64, new_rows=4, max_cap=754)
    with pytest.raises(rkv.RkvError):
        rkv.rkv_state_init_host(ecfg, 750, 753, 0)


def test_capacity_beyond_the_ring_is_rejected(rkv):
    """A stream capacity above cfg.max_cap fails at state set-up, and a ring
    with fewer slots than cfg.max_cap fails every call that takes it, so no
    state can name a row the ring lacks (voxtral.c explainer, section 二: the
    buffer's capacity kv_cache_max bounds every row index)."""
    ccfg = good_cfg(rkv, mode=rkv.RKV_MODE_COMPACT, max_cap=9000)
    with pytest.raises(rkv.RkvError) as e:
        rkv.rkv_state_init_host(ccfg, 8192, 9216, 0)          # cap 9216 > max_cap 9000
    assert e.value.status == rkv.RKV_ESTATE
    assert rkv.rkv_state_init_host(ccfg, 8192, 9000, 0)["cap"][0] == 9000
    ecfg = good_cfg(rkv, mode=rkv.RKV_MODE_ENC_CHUNK, num_q_heads=20, num_kv_heads=20,
                    head_dim=64, new_rows=4, max_cap=753)
    with pytest.raises(rkv.RkvError) as e:
        rkv.rkv_state_init_host(ecfg, 750, 754, 0)
    assert e.value.status == rkv.RKV_ESTATE
    unset = good_cfg(rkv, max_cap=0)
    with pytest.raises(rkv.RkvError) as e:
        rkv.rkv_state_init_host(unset, 375, 375, 0)
    assert e.value.status == rkv.RKV_EINVAL
    W = np.full(unset.num_streams, 375, np.int32)
    O = np.zeros(unset.num_streams, np.int64)
    assert call(rkv, "rkv_state_init", ctypes.byref(unset), ctypes.c_void_p(FAKE), W.ctypes.data,
                W.ctypes.data, O.ctypes.data, None) == rkv.RKV_EINVAL
    # a 374-slot ring for states of capacity up to 375
    cfg = good_cfg(rkv)
    short = fake_view(rkv, slots=374)
    F, N = ctypes.c_void_p(FAKE), None
    c, k = ctypes.byref(cfg), ctypes.byref(short)
    assert call(rkv, "rkv_append", c, F, k, F, F, N) == rkv.RKV_ESTATE
    assert call(rkv, "rkv_update_step", c, F, k, F, F, N) == rkv.RKV_ESTATE
    assert call(rkv, "rkv_roll_rebase", c, F, k, N) == rkv.RKV_ESTATE
    assert call(rkv, "rkv_decode_attn", c, F, k, F, F, N, 0, N) == rkv.RKV_ESTATE
    assert call(rkv, "rkv_decode_step", c, F, k, F, F, F, F, N, 0, N) == rkv.RKV_ESTATE
    PL = ctypes.c_void_p(FAKE + 0x100000)
    assert call(rkv, "rkv_decode_step_pipelined", c, F, F, PL, k, F, F, F, F, N, 0,
                N) == rkv.RKV_ESTATE
    assert call(rkv, "rkv_decode_attn_pipelined", c, F, F, PL, k, F, F, N, 0,
                N) == rkv.RKV_ESTATE
    comp = good_cfg(rkv, mode=rkv.RKV_MODE_COMPACT)
    assert call(rkv, "rkv_compact", ctypes.byref(comp), F, k, N) == rkv.RKV_ESTATE
    enc = good_cfg(rkv, mode=rkv.RKV_MODE_ENC_CHUNK, num_q_heads=20, num_kv_heads=20,
                   head_dim=64, new_rows=4)
    assert call(rkv, "rkv_encoder_chunk_attn", ctypes.byref(enc), F, k, F, F, F, F, N, 0,
                N) == rkv.RKV_ESTATE
    # the same ring with max_cap unset: rejected as an invalid configuration
    assert call(rkv, "rkv_append", ctypes.byref(unset), F, ctypes.byref(fake_view(rkv)), F, F,
                N) == rkv.RKV_EINVAL
    assert rkv.rkv_last_hip_error() == 0


def test_workspace_sizes(rkv):
    # a split call's workspace: one uint32 merge counter per (layer, stream,
    # kv head) item padded to 256 bytes, then the float32 partials
    part = (16 + 8 * 128) * 4
    # 36 x 64 x 2 = 4608 items: no split needed
    assert rkv.rkv_workspace_bytes(good_cfg(rkv, num_streams=64, num_layers=36), 375) == 0
    # one stream, one layer, W = 375: splits of 256 keys at least, so none
    one = dict(num_streams=1, num_layers=1)
    assert rkv.rkv_workspace_bytes(good_cfg(rkv, **one), 375) == 0
    # ... with 2048 keys: 8 ranges (2 items, 2048 / 256 keys each)
    assert rkv.rkv_workspace_bytes(good_cfg(rkv, **one), 2048) == 256 + 2 * 8 * part
    # re-base every position with the residual: splits of about 48 keys,
    # round(375 / 48) = 8, round(250 / 48) = 5
    comp = good_cfg(rkv, rebase_chunk=1, flags=rkv.RKV_F_COMPENSATED, **one)
    assert rkv.rkv_workspace_bytes(comp, 375) == 256 + 2 * 8 * part
    assert rkv.rkv_workspace_bytes(comp, 250) == 256 + 2 * 5 * part
    # an explicit count is kept up to one split per 16 slots and 64 in all
    assert rkv.rkv_workspace_bytes(good_cfg(rkv, num_splits=6, **one), 375) == \
        256 + 2 * 6 * part
    assert rkv.rkv_workspace_bytes(good_cfg(rkv, num_splits=100, **one), 8192) == \
        256 + 2 * 64 * part
    # the separate merge launch keeps the same layout
    sep = good_cfg(rkv, num_splits=6, flags=rkv.RKV_F_MERGE_LAUNCH, **one)
    assert rkv.rkv_workspace_bytes(sep, 375) == 256 + 2 * 6 * part
    # 130 items: the counters take 520 bytes, padded to 768
    many = good_cfg(rkv, num_streams=65, num_layers=1, num_splits=2)
    assert rkv.rkv_workspace_bytes(many, 375) == 768 + 130 * 2 * part
    assert rkv.rkv_workspace_bytes(good_cfg(rkv, head_dim=3), 375) == 0
    assert rkv.rkv_validate_cfg(good_cfg(rkv, flags=rkv.RKV_F_MERGE_LAUNCH)) == rkv.RKV_OK
    assert rkv.rkv_validate_cfg(good_cfg(rkv, flags=16)) == rkv.RKV_EUNSUPPORTED


FAKE = 0x10000           # never dereferenced: every call below fails validation
MISALIGNED = 0x10008


def fake_view(rkv, k=FAKE, lo=None, slot_stride=128, slots=375):
    return rkv.rkv_kv_view(k, FAKE, lo, 2 * 4 * 375 * 128 * 0 + 4 * 2 * 375 * 128,
                           2 * 375 * 128, 375 * 128, slot_stride, slots, 0)


def call(rkv, name, *args):
    return getattr(rkv.lib(), name)(*args)


def test_calls_reject_bad_arguments_without_a_device(rkv):
    cfg = good_cfg(rkv)
    c = ctypes.byref(cfg)
    kv = fake_view(rkv)
    F = ctypes.c_void_p(FAKE)
    N = None
    M = ctypes.c_void_p(MISALIGNED)
    assert call(rkv, "rkv_advance", c, N, F, N) == rkv.RKV_EINVAL
    assert call(rkv, "rkv_advance", N, F, F, N) == rkv.RKV_EINVAL
    assert call(rkv, "rkv_append", c, F, ctypes.byref(kv), N, F, N) == rkv.RKV_EINVAL
    assert call(rkv, "rkv_append", c, F, ctypes.byref(kv), M, F, N) == rkv.RKV_EALIGN
    assert call(rkv, "rkv_append", c, F, N, F, F, N) == rkv.RKV_EINVAL
    assert call(rkv, "rkv_update_step", c, F, ctypes.byref(kv), N, F, N) == rkv.RKV_EINVAL
    assert call(rkv, "rkv_update_step", c, F, ctypes.byref(kv), F, M, N) == rkv.RKV_EALIGN
    assert call(rkv, "rkv_update_step", c, N, ctypes.byref(kv), F, F, N) == rkv.RKV_EINVAL
    assert call(rkv, "rkv_update_step", c, F, N, F, F, N) == rkv.RKV_EINVAL
    # read-only pipelined attention: distinct plan buffers, no encoder mode
    PL2 = ctypes.c_void_p(FAKE + 0x100000)
    assert call(rkv, "rkv_decode_attn_pipelined", c, F, F, F, ctypes.byref(kv), F, F, N, 0,
                N) == rkv.RKV_EINVAL
    assert call(rkv, "rkv_decode_attn_pipelined", c, N, F, PL2, ctypes.byref(kv), F, F, N, 0,
                N) == rkv.RKV_EINVAL
    assert call(rkv, "rkv_decode_attn_pipelined", c, F, F, PL2, ctypes.byref(kv), M, F, N, 0,
                N) == rkv.RKV_EALIGN
    enc = rkv.make_cfg(2, 1, num_q_heads=4, num_kv_heads=4, head_dim=64,
                       mode=rkv.RKV_MODE_ENC_CHUNK, new_rows=4)
    assert call(rkv, "rkv_decode_attn_pipelined", ctypes.byref(enc), F, F, PL2,
                ctypes.byref(kv), F, F, N, 0, N) == rkv.RKV_EINVAL
    bad_stride = fake_view(rkv, slot_stride=100)
    assert call(rkv, "rkv_roll_rebase", c, F, ctypes.byref(bad_stride), N) == rkv.RKV_EINVAL
    odd_stride = fake_view(rkv, slot_stride=132)
    assert call(rkv, "rkv_roll_rebase", c, F, ctypes.byref(odd_stride), N) == rkv.RKV_EALIGN
    mis = fake_view(rkv, k=MISALIGNED)
    assert call(rkv, "rkv_roll_rebase", c, F, ctypes.byref(mis), N) == rkv.RKV_EALIGN
    assert call(rkv, "rkv_roll_rebase", c, N, ctypes.byref(kv), N) == rkv.RKV_EINVAL
    # mode mismatches
    assert call(rkv, "rkv_compact", c, F, ctypes.byref(kv), N) == rkv.RKV_EINVAL
    assert call(rkv, "rkv_encoder_chunk_attn", c, F, ctypes.byref(kv), F, F, F, F, N, 0,
                N) == rkv.RKV_EINVAL
    # compensated needs k_lo
    ccfg = good_cfg(rkv, flags=rkv.RKV_F_COMPENSATED)
    assert call(rkv, "rkv_roll_rebase", ctypes.byref(ccfg), F, ctypes.byref(kv),
                N) == rkv.RKV_EINVAL
    # decode: missing workspace when the key range is split
    one = good_cfg(rkv, num_streams=1, num_layers=1, num_splits=6)
    assert call(rkv, "rkv_decode_attn", ctypes.byref(one), F, ctypes.byref(kv), F, F, N, 0,
                N) == rkv.RKV_ESPACE
    assert call(rkv, "rkv_decode_step", ctypes.byref(one), F, ctypes.byref(kv), F, F, F, F,
                F, 16, N) == rkv.RKV_ESPACE
    assert call(rkv, "rkv_decode_attn", c, F, ctypes.byref(kv), M, F, N, 0,
                N) == rkv.RKV_EALIGN
    assert call(rkv, "rkv_decode_step", c, F, ctypes.byref(kv), F, F, N, F, N, 0,
                N) == rkv.RKV_EINVAL
    # pipelined step: the plan read and the plan written must be distinct buffers
    PL = ctypes.c_void_p(FAKE + 0x100000)
    assert call(rkv, "rkv_decode_step_pipelined", c, F, F, F, ctypes.byref(kv), F, F, F, F, N,
                0, N) == rkv.RKV_EINVAL
    assert call(rkv, "rkv_decode_step_pipelined", c, F, F, ctypes.c_void_p(FAKE + 64),
                ctypes.byref(kv), F, F, F, F, N, 0, N) == rkv.RKV_EINVAL
    assert call(rkv, "rkv_decode_step_pipelined", c, N, F, PL, ctypes.byref(kv), F, F, F, F, N,
                0, N) == rkv.RKV_EINVAL
    assert call(rkv, "rkv_decode_step_pipelined", c, F, F, ctypes.c_void_p(FAKE + 0x100008),
                ctypes.byref(kv), F, F, F, F, N, 0, N) == rkv.RKV_EALIGN
    assert call(rkv, "rkv_decode_step_pipelined", c, ctypes.c_void_p(FAKE + 4), F, PL,
                ctypes.byref(kv), F, F, F, F, N, 0, N) == rkv.RKV_EALIGN
    # device state init: bad host arrays and mismatched streams fail before any copy
    W = np.full(cfg.num_streams, 375, np.int32)
    O = np.zeros(cfg.num_streams, np.int64)
    assert call(rkv, "rkv_state_init", c, N, W.ctypes.data, W.ctypes.data, O.ctypes.data,
                N) == rkv.RKV_EINVAL
    assert call(rkv, "rkv_state_init", c, F, N, W.ctypes.data, O.ctypes.data,
                N) == rkv.RKV_EINVAL
    assert call(rkv, "rkv_state_init", c, ctypes.c_void_p(FAKE + 4), W.ctypes.data,
                W.ctypes.data, O.ctypes.data, N) == rkv.RKV_EALIGN
    W1 = W + 1
    assert call(rkv, "rkv_state_init", c, F, W.ctypes.data, W1.ctypes.data, O.ctypes.data,
                N) == rkv.RKV_ESTATE
    assert rkv.rkv_last_hip_error() == 0


def test_reset_streams_rejects_bad_arguments_without_a_device(rkv):
    cfg = good_cfg(rkv)
    c = ctypes.byref(cfg)
    F = ctypes.c_void_p(FAKE)
    N = None
    S = cfg.num_streams
    st = np.array([0, S - 1], np.int32)
    org = np.array([0, 5], np.int64)
    reset = lambda *a: call(rkv, "rkv_reset_streams", *a)
    assert reset(N, F, N, 2, st.ctypes.data, org.ctypes.data, N) == rkv.RKV_EINVAL
    assert reset(c, N, N, 2, st.ctypes.data, org.ctypes.data, N) == rkv.RKV_EINVAL
    assert reset(c, F, N, -1, st.ctypes.data, org.ctypes.data, N) == rkv.RKV_EINVAL
    assert reset(c, F, N, 2, N, org.ctypes.data, N) == rkv.RKV_EINVAL
    assert reset(c, F, N, 2, st.ctypes.data, N, N) == rkv.RKV_EINVAL
    bad = np.array([0, S], np.int32)
    assert reset(c, F, N, 2, bad.ctypes.data, org.ctypes.data, N) == rkv.RKV_EINVAL
    neg = np.array([-1, 0], np.int32)
    assert reset(c, F, N, 2, neg.ctypes.data, org.ctypes.data, N) == rkv.RKV_EINVAL
    before = np.array([0, -3], np.int64)
    assert reset(c, F, N, 2, st.ctypes.data, before.ctypes.data, N) == rkv.RKV_ESTATE
    assert reset(c, ctypes.c_void_p(FAKE + 4), N, 2, st.ctypes.data, org.ctypes.data,
                 N) == rkv.RKV_EALIGN
    assert reset(c, F, ctypes.c_void_p(FAKE + 8), 2, st.ctypes.data, org.ctypes.data,
                 N) == rkv.RKV_EALIGN
    # nothing to restart: no launch, no device needed
    assert reset(c, F, N, 0, N, N, N) == rkv.RKV_OK
    assert rkv.rkv_last_hip_error() == 0


def test_fp16_cache_flag(rkv):
    ok = good_cfg(rkv, flags=rkv.RKV_F_KV_FP16)
    assert rkv.lib().rkv_validate_cfg(ctypes.byref(ok)) == rkv.RKV_OK
    both = good_cfg(rkv, flags=rkv.RKV_F_KV_FP16 | rkv.RKV_F_COMPENSATED)
    assert rkv.lib().rkv_validate_cfg(ctypes.byref(both)) == rkv.RKV_OK
    comp = rkv.make_cfg(2, 1, mode=rkv.RKV_MODE_COMPACT, flags=rkv.RKV_F_KV_FP16)
    assert rkv.lib().rkv_validate_cfg(ctypes.byref(comp)) == rkv.RKV_OK
    enc = rkv.make_cfg(2, 1, num_q_heads=4, num_kv_heads=4, head_dim=64,
                       mode=rkv.RKV_MODE_ENC_CHUNK, new_rows=4, flags=rkv.RKV_F_KV_FP16)
    assert rkv.lib().rkv_validate_cfg(ctypes.byref(enc)) == rkv.RKV_EUNSUPPORTED
    unknown = good_cfg(rkv, flags=1 << 4)
    assert rkv.lib().rkv_validate_cfg(ctypes.byref(unknown)) == rkv.RKV_EUNSUPPORTED


def test_encoder_step_sizes_and_validation(rkv):
    S, L, H, d, F, slots, ffn = 2, 3, 4, 64, 4, 24, 1024
    hidden = H * d
    cfg = rkv.make_cfg(S, L, num_q_heads=H, num_kv_heads=H, head_dim=d,
                       mode=rkv.RKV_MODE_ENC_CHUNK, new_rows=F, max_cap=slots)
    ec = rkv.make_encoder_cfg(ffn=ffn, norm_eps=1e-5)
    # g1, wq, wk, wv, wo, g2, w1, w2 in bfloat16
    assert rkv.rkv_encoder_layer_weight_bytes(cfg, ec) == 2 * (2 * hidden + 4 * hidden ** 2
                                                                + 2 * hidden * ffn)
    ws = rkv.rkv_encoder_step_workspace_bytes(cfg, ec, slots)
    assert ws >= 2 * S * F * (5 * hidden + ffn)
    bad = [rkv.make_encoder_cfg(ffn=48), rkv.make_encoder_cfg(ffn=96), rkv.make_encoder_cfg(ffn=0),
           rkv.make_encoder_cfg(norm_eps=-1.0), rkv.make_encoder_cfg(norm_eps=float("nan"))]
    for b in bad:
        assert rkv.rkv_encoder_layer_weight_bytes(cfg, b) == 0
        assert rkv.rkv_encoder_step_workspace_bytes(cfg, b, slots) == 0
    dec = good_cfg(rkv)
    assert rkv.rkv_encoder_layer_weight_bytes(dec, ec) == 0
    for heads, dim in ((1, 32), (65, 64)):      # hidden 32: not a multiple of 64; 4160 > 4096
        wide = rkv.make_cfg(S, L, num_q_heads=heads, num_kv_heads=heads, head_dim=dim,
                            mode=rkv.RKV_MODE_ENC_CHUNK, new_rows=F)
        if rkv.rkv_validate_cfg(wide) == rkv.RKV_OK:
            assert rkv.rkv_encoder_layer_weight_bytes(wide, ec) == 0
    assert rkv.rkv_encoder_step_workspace_bytes(cfg, ec, 0) == 0
    kv = rkv.rkv_kv_view(FAKE, FAKE + 0x1000000, None, S * H * slots * d, H * slots * d,
                         slots * d, d, slots, 0)
    c, e, k = ctypes.byref(cfg), ctypes.byref(ec), ctypes.byref(kv)
    P, W, X, WS = (ctypes.c_void_p(FAKE + o) for o in (0x2000000, 0x3000000, 0x4000000,
                                                       0x5000000))
    N = None
    step = lambda *a: call(rkv, "rkv_encoder_step", *a)
    assert step(c, e, N, k, W, X, WS, ws, N) == rkv.RKV_EINVAL
    assert step(c, None, P, k, W, X, WS, ws, N) == rkv.RKV_EINVAL
    assert step(c, e, P, k, W, ctypes.c_void_p(FAKE + 0x4000008), WS, ws, N) == rkv.RKV_EALIGN
    assert step(c, e, P, k, ctypes.c_void_p(FAKE + 0x3000004), X, WS, ws, N) == rkv.RKV_EALIGN
    assert step(c, e, P, k, W, X, WS, ws - 1, N) == rkv.RKV_ESPACE
    f32 = rkv.make_cfg(S, L, num_q_heads=H, num_kv_heads=H, head_dim=d,
                       mode=rkv.RKV_MODE_ENC_CHUNK, new_rows=F, flags=rkv.RKV_F_OUT_F32,
                       max_cap=slots)
    assert step(ctypes.byref(f32), e, P, k, W, X, WS, ws, N) == rkv.RKV_EUNSUPPORTED
    assert step(ctypes.byref(dec), e, P, k, W, X, WS, ws, N) == rkv.RKV_EINVAL
    assert step(c, ctypes.byref(bad[0]), P, k, W, X, WS, ws, N) == rkv.RKV_EINVAL
    assert rkv.rkv_last_hip_error() == 0


def test_tcond_sizes_and_validation(rkv):
    assert ctypes.sizeof(rkv.rkv_tcond_cfg) == 32
    L, C = 2, 3
    cfg = good_cfg(rkv, num_layers=L)                       # 16 x 128 = 2048 features
    tc = rkv.make_tcond_cfg(L, 2048, dim=256, num_conds=C, max_frame_len=8)
    n = np.array([6, 3, 2], np.int32)
    f = np.array([4, 6, 8], np.int32)
    F = ctypes.c_void_p(FAKE)
    M = ctypes.c_void_p(MISALIGNED)
    N = None
    prep = lambda t, nn, ff, a, b, c: call(rkv, "rkv_tcond_prepare", t, nn, ff, a, b, c, N)
    t = ctypes.byref(tc)
    assert prep(N, n.ctypes.data, f.ctypes.data, F, F, F) == rkv.RKV_EINVAL
    assert prep(t, N, f.ctypes.data, F, F, F) == rkv.RKV_EINVAL
    assert prep(t, n.ctypes.data, f.ctypes.data, F, F, N) == rkv.RKV_EINVAL
    assert prep(t, n.ctypes.data, f.ctypes.data, M, F, F) == rkv.RKV_EALIGN
    assert prep(t, n.ctypes.data, f.ctypes.data, F, F, M) == rkv.RKV_EALIGN
    bad_f = np.array([4, 9, 8], np.int32)                    # beyond the 9-row table
    assert prep(t, n.ctypes.data, bad_f.ctypes.data, F, F, F) == rkv.RKV_EINVAL
    bad_n = np.array([6, -1, 2], np.int32)
    assert prep(t, bad_n.ctypes.data, f.ctypes.data, F, F, F) == rkv.RKV_EINVAL
    for kw in (dict(dim=255), dict(dim=0), dict(dim=2048), dict(num_conds=0),
               dict(num_conds=65), dict(hidden=12), dict(max_frame_len=-1)):
        args = dict(num_layers=L, hidden=2048, dim=256, num_conds=C, max_frame_len=8)
        args.update(kw)
        bad = rkv.make_tcond_cfg(**args)
        assert prep(ctypes.byref(bad), n.ctypes.data, f.ctypes.data, F, F, F) == rkv.RKV_EINVAL
    mod = lambda c, t_, a, b, o: call(rkv, "rkv_tcond_modulate", c, t_, a, b, o, N)
    c = ctypes.byref(cfg)
    assert mod(c, t, F, N, F) == rkv.RKV_EINVAL
    assert mod(c, t, F, F, M) == rkv.RKV_EALIGN
    assert mod(c, t, M, F, F) == rkv.RKV_EALIGN
    other = rkv.make_tcond_cfg(L + 1, 2048, dim=256, num_conds=C)
    assert mod(c, ctypes.byref(other), F, F, F) == rkv.RKV_EINVAL
    narrow = rkv.make_tcond_cfg(L, 1024, dim=256, num_conds=C)
    assert mod(c, ctypes.byref(narrow), F, F, F) == rkv.RKV_EINVAL
    assert mod(N, t, F, F, F) == rkv.RKV_EINVAL
    # the decode step with the modulation applied as it stores its output
    kv = fake_view(rkv)
    k = ctypes.byref(kv)
    fused = lambda c_, t_, a, b: call(rkv, "rkv_decode_step_pipelined_tcond", c_, t_, a, b, F, F,
                                      ctypes.c_void_p(FAKE + 0x100000), k, F, F, F, F, N, 0, N)
    assert fused(c, t, F, N) == rkv.RKV_EINVAL                 # no stream conditions
    assert fused(c, t, M, F) == rkv.RKV_EALIGN                 # misaligned vectors
    assert fused(c, ctypes.byref(other), F, F) == rkv.RKV_EINVAL
    assert fused(c, ctypes.byref(narrow), F, F) == rkv.RKV_EINVAL
    assert fused(c, N, F, F) == rkv.RKV_EINVAL
    enc = rkv.make_cfg(2, L, num_q_heads=16, num_kv_heads=16, head_dim=128,
                       mode=rkv.RKV_MODE_ENC_CHUNK, new_rows=4, max_cap=375)
    assert fused(ctypes.byref(enc), t, F, F) == rkv.RKV_EINVAL  # decoder modes only
    assert rkv.rkv_last_hip_error() == 0


def test_no_alloc_step_rejects_what_its_array_cannot_hold(rkv):
    """rkv_decode_step_noalloc checks every argument, and the size of the split
    partials against the library's array, before any HIP call."""
    F, N = ctypes.c_void_p(FAKE), None
    M = ctypes.c_void_p(MISALIGNED)
    cfg = good_cfg(rkv)
    kv = fake_view(rkv)
    c, k = ctypes.byref(cfg), ctypes.byref(kv)
    f = rkv.lib().rkv_decode_step_noalloc
    assert f(c, N, k, F, F, F, F, N) == rkv.RKV_EINVAL
    assert f(c, F, k, M, F, F, F, N) == rkv.RKV_EALIGN
    assert f(c, F, k, F, N, F, F, N) == rkv.RKV_EINVAL
    assert f(N, F, k, F, F, F, F, N) == rkv.RKV_EINVAL
    # one layer of 64 streams (128 items), 23 splits of a 375-slot ring: 12.2 MB
    # of partials (128 x 23 x 4,160 bytes) fit beside the array's merge counters ...
    fits = good_cfg(rkv, num_streams=64, num_layers=1, num_splits=23)
    assert rkv.rkv_workspace_bytes(fits, 375) == 512 + 128 * 23 * 4160
    assert 128 * 23 * 4160 < rkv.RKV_NOALLOC_SCRATCH_BYTES - 4 * rkv.RKV_NOALLOC_MAX_SPLIT_ITEMS
    # ... 64 splits of an 8192-slot ring (34 MB) do not
    big = good_cfg(rkv, num_streams=64, num_layers=1, num_splits=64, max_cap=8192)
    big_kv = fake_view(rkv, slots=8192)
    assert rkv.rkv_workspace_bytes(big, 8192) > rkv.RKV_NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(big), F, ctypes.byref(big_kv), F, F, F, F, N) == rkv.RKV_ESPACE
    assert rkv.rkv_last_hip_error() == 0
