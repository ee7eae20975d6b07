"""ctypes binding of librkv.so (declared in include/rkv.h).

Argument marshalling only: torch tensors are passed as device pointers and the
current torch HIP stream is passed as the stream; every step of the path runs
in the library's HIP kernels.  There is no fallback: if the library is not
built, importing this module raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

# RKV_LIBRARY names another build of the same sources (the host-sanitizer
# test loads an instrumented copy); by default the in-tree librkv.so.
_LIB_PATH = os.environ.get("RKV_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "librkv.so")

RKV_OK = 0
RKV_EINVAL = -1
RKV_EUNSUPPORTED = -2
RKV_EALIGN = -3
RKV_ESTATE = -4
RKV_EHIP = -5
RKV_ESPACE = -6

RKV_MODE_REBASE = 0
RKV_MODE_COMPACT = 1
RKV_MODE_ENC_CHUNK = 2

RKV_F_COMPENSATED = 1
RKV_F_OUT_F32 = 2
RKV_F_KV_FP16 = 4
RKV_F_MERGE_LAUNCH = 8

RKV_MAX_NEW_ROWS = 8
RKV_MAX_HEAD_DIM = 128
RKV_NOALLOC_SCRATCH_BYTES = 16 << 20
RKV_NOALLOC_MAX_SPLIT_ITEMS = 16384

# Entry points declared in include/rkv.h (checked by the ABI tests).
ENTRY_POINTS = (
    "rkv_version", "rkv_strerror", "rkv_last_hip_error", "rkv_validate_cfg",
    "rkv_state_init_host", "rkv_state_advance_host", "rkv_state_init", "rkv_workspace_bytes", "rkv_advance", "rkv_append",
    "rkv_roll_rebase", "rkv_update_step", "rkv_compact", "rkv_decode_attn", "rkv_decode_step",
    "rkv_decode_step_noalloc", "rkv_decode_step_pipelined", "rkv_decode_attn_pipelined",
    "rkv_encoder_chunk_attn", "rkv_reset_streams", "rkv_restart_step",
    "rkv_mel_filters_host", "rkv_mel_step",
    "rkv_encoder_layer_weight_bytes", "rkv_encoder_step_workspace_bytes", "rkv_encoder_step",
    "rkv_tcond_delay_tokens", "rkv_tcond_prepare", "rkv_tcond_modulate",
    "rkv_decode_step_pipelined_tcond",
)

RKV_TCOND_MAX_CONDS = 64
RKV_TCOND_MAX_DIM = 1024

RKV_STREAM_MAX_DECODE_KV = 2000
RKV_RESTART_NONE = 0
RKV_RESTART_EOS = 1
RKV_RESTART_KV_OVERFLOW = 2
RKV_RESTART_NONTEXT_RUN = 3
RKV_RESTART_STALL = 4


class RkvError(RuntimeError):
    def __init__(self, fn, status):
        msg = f"{fn} failed: {status} ({strerror(status)})"
        if status == RKV_EHIP:
            msg += f", hipError {lib().rkv_last_hip_error()}"
        super().__init__(msg)
        self.status = status


class rkv_cfg(ctypes.Structure):
    _fields_ = [
        ("num_streams", ctypes.c_int32), ("num_layers", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("mode", ctypes.c_int32),
        ("rebase_chunk", ctypes.c_int32), ("new_rows", ctypes.c_int32),
        ("flags", ctypes.c_uint32), ("num_splits", ctypes.c_int32),
        ("rope_base", ctypes.c_double), ("softmax_scale", ctypes.c_float),
        ("max_cap", ctypes.c_int32),
    ]


class rkv_kv_view(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("k_lo", ctypes.c_void_p),
        ("layer_stride", ctypes.c_int64), ("stream_stride", ctypes.c_int64),
        ("head_stride", ctypes.c_int64), ("slot_stride", ctypes.c_int64),
        ("slots", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


class rkv_encoder_cfg(ctypes.Structure):
    _fields_ = [("ffn", ctypes.c_int32), ("norm_eps", ctypes.c_float),
                ("reserved", ctypes.c_int32 * 2)]


class rkv_tcond_cfg(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("dim", ctypes.c_int32), ("num_conds", ctypes.c_int32),
                ("max_frame_len", ctypes.c_int32), ("reserved", ctypes.c_int32 * 3)]


class rkv_mel_cfg(ctypes.Structure):
    _fields_ = [
        ("num_streams", ctypes.c_int32), ("n_fft", ctypes.c_int32), ("hop", ctypes.c_int32),
        ("n_mels", ctypes.c_int32), ("samples_per_step", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class rkv_restart_cfg(ctypes.Structure):
    _fields_ = [
        ("max_decode_kv", ctypes.c_int64), ("eos_token", ctypes.c_int32),
        ("text_token_min", ctypes.c_int32), ("nontext_run", ctypes.c_int32),
        ("stall_steps", ctypes.c_int32),
    ]


RESTART_STATE_DTYPE = np.dtype([
    ("decode_len", "<i8"), ("restarts", "<i8"), ("nontext", "<i4"), ("idle", "<i4"),
])

STATE_DTYPE = np.dtype([
    ("t", "<i8"), ("origin", "<i8"), ("pos_offset", "<i8"),
    ("len", "<i4"), ("window", "<i4"), ("cap", "<i4"), ("reserved", "<i4", (3,)),
])

PLAN_DTYPE = np.dtype([
    ("t", "<i8"), ("pos", "<i8"), ("pos_offset", "<i8"), ("first_pos", "<i8"),
    ("evict_pos", "<i8"), ("slot", "<i4"), ("n_valid", "<i4"), ("rebase_delta", "<i4"),
    ("compact_drop", "<i4"), ("evict_slot", "<i4"), ("window", "<i4"), ("cap", "<i4"),
    ("new_rows", "<i4"), ("reserved", "<i4", (14,)),
    ("rope_new", "<f8", (RKV_MAX_NEW_ROWS, 2, RKV_MAX_HEAD_DIM // 2)),
    ("rope_delta", "<f8", (2, RKV_MAX_HEAD_DIM // 2)),
])
assert STATE_DTYPE.itemsize == 48 and PLAN_DTYPE.itemsize == 9344

_lib = None


def lib():
    """The loaded librkv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is not built; run `python -m rolling_window_kv_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        pc = ctypes.POINTER(rkv_cfg)
        pk = ctypes.POINTER(rkv_kv_view)
        sig = {
            "rkv_version": ([], ctypes.c_int),
            "rkv_strerror": ([ctypes.c_int], ctypes.c_char_p),
            "rkv_last_hip_error": ([], ctypes.c_int),
            "rkv_validate_cfg": ([pc], ctypes.c_int),
            "rkv_state_init_host": ([pc, vp, vp, vp, vp], ctypes.c_int),
            "rkv_state_advance_host": ([pc, vp, ctypes.c_int64], ctypes.c_int),
            "rkv_state_init": ([pc, vp, vp, vp, vp, vp], ctypes.c_int),
            "rkv_workspace_bytes": ([pc, i32], sz),
            "rkv_advance": ([pc, vp, vp, vp], ctypes.c_int),
            "rkv_append": ([pc, vp, pk, vp, vp, vp], ctypes.c_int),
            "rkv_roll_rebase": ([pc, vp, pk, vp], ctypes.c_int),
            "rkv_update_step": ([pc, vp, pk, vp, vp, vp], ctypes.c_int),
            "rkv_compact": ([pc, vp, pk, vp], ctypes.c_int),
            "rkv_decode_attn": ([pc, vp, pk, vp, vp, vp, sz, vp], ctypes.c_int),
            "rkv_decode_step": ([pc, vp, pk, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
            "rkv_decode_step_noalloc": ([pc, vp, pk, vp, vp, vp, vp, vp], ctypes.c_int),
            "rkv_decode_step_pipelined": ([pc, vp, vp, vp, pk, vp, vp, vp, vp, vp, sz, vp],
                                          ctypes.c_int),
            "rkv_decode_attn_pipelined": ([pc, vp, vp, vp, pk, vp, vp, vp, sz, vp],
                                          ctypes.c_int),
            "rkv_encoder_chunk_attn": ([pc, vp, pk, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
            "rkv_reset_streams": ([pc, vp, vp, i32, vp, vp, vp], ctypes.c_int),
            "rkv_restart_step": ([ctypes.POINTER(rkv_restart_cfg), vp, i32, vp, vp, vp],
                                 ctypes.c_int),
            "rkv_mel_filters_host": ([ctypes.POINTER(rkv_mel_cfg), ctypes.c_double, vp],
                                     ctypes.c_int),
            "rkv_mel_step": ([ctypes.POINTER(rkv_mel_cfg), vp, vp, vp, vp, vp, vp],
                             ctypes.c_int),
            "rkv_encoder_layer_weight_bytes": ([pc, ctypes.POINTER(rkv_encoder_cfg)], sz),
            "rkv_encoder_step_workspace_bytes": ([pc, ctypes.POINTER(rkv_encoder_cfg), i32], sz),
            "rkv_encoder_step": ([pc, ctypes.POINTER(rkv_encoder_cfg), vp, pk, vp, vp, vp, sz, vp],
                                 ctypes.c_int),
            "rkv_tcond_delay_tokens": ([i32, i32, vp, vp], ctypes.c_int),
            "rkv_tcond_prepare": ([ctypes.POINTER(rkv_tcond_cfg), vp, vp, vp, vp, vp, vp],
                                  ctypes.c_int),
            "rkv_tcond_modulate": ([pc, ctypes.POINTER(rkv_tcond_cfg), vp, vp, vp, vp],
                                   ctypes.c_int),
            "rkv_decode_step_pipelined_tcond": (
                [pc, ctypes.POINTER(rkv_tcond_cfg), vp, vp, vp, vp, vp, pk, vp, vp, vp, vp, vp,
                 sz, vp], ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def lib_path():
    return _LIB_PATH


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def make_cfg(num_streams, num_layers, num_q_heads=16, num_kv_heads=2, head_dim=128,
             mode=RKV_MODE_REBASE, rebase_chunk=1, new_rows=1, flags=0, num_splits=0,
             rope_base=1e6, softmax_scale=0.0, max_cap=0) -> rkv_cfg:
    """max_cap: ring rows per (layer, stream, head); 0 leaves it to :class:`Cache`,
    which declares its own slot count."""
    return rkv_cfg(num_streams, num_layers, num_q_heads, num_kv_heads, head_dim, mode,
                   rebase_chunk, new_rows, flags, num_splits, rope_base, softmax_scale,
                   max_cap)


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, rc):
    if rc != RKV_OK:
        raise RkvError(fn, rc)


def kv_view(k, v, k_lo=None) -> rkv_kv_view:
    """View of cache tensors shaped [L, S, Hkv, slots, d] (bf16, last dim contiguous)."""
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("K and V must have the same shape and strides")
    if k.stride(-1) != 1:
        raise ValueError("head_dim must be contiguous")
    if k_lo is not None and (k_lo.shape != k.shape or k_lo.stride() != k.stride()):
        raise ValueError("k_lo must match K")
    st = k.stride()
    return rkv_kv_view(k.data_ptr(), v.data_ptr(), None if k_lo is None else k_lo.data_ptr(),
                       st[0], st[1], st[2], st[3], k.shape[3], 0)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def rkv_version() -> int:
    return lib().rkv_version()


def strerror(status) -> str:
    return lib().rkv_strerror(int(status)).decode()


rkv_strerror = strerror


def rkv_last_hip_error() -> int:
    return lib().rkv_last_hip_error()


def rkv_validate_cfg(cfg) -> int:
    return lib().rkv_validate_cfg(ctypes.byref(cfg))


def _state_args(cfg, window, cap, origin):
    S = cfg.num_streams
    w = np.ascontiguousarray(np.broadcast_to(np.asarray(window, np.int32), (S,)))
    c = np.ascontiguousarray(np.broadcast_to(np.asarray(cap, np.int32), (S,)))
    o = np.ascontiguousarray(np.broadcast_to(np.asarray(origin, np.int64), (S,)))
    return w, c, o


def rkv_state_init(cfg, state, window, cap, origin, stream=None):
    """Write the initial per-stream states into the device tensor `state`
    (S * 48 bytes); returns once the copy is done."""
    w, c, o = _state_args(cfg, window, cap, origin)
    _check("rkv_state_init", lib().rkv_state_init(ctypes.byref(cfg), _ptr(state), w.ctypes.data,
                                                  c.ctypes.data, o.ctypes.data, _stream(stream)))


def rkv_state_init_host(cfg, window, cap, origin) -> np.ndarray:
    """Per-stream initial states as a STATE_DTYPE array (host)."""
    S = cfg.num_streams
    w, c, o = _state_args(cfg, window, cap, origin)
    out = np.zeros(S, STATE_DTYPE)
    rc = lib().rkv_state_init_host(ctypes.byref(cfg), w.ctypes.data, c.ctypes.data,
                                   o.ctypes.data, out.ctypes.data)
    _check("rkv_state_init_host", rc)
    return out


def rkv_state_advance_host(cfg, states, steps):
    """Advance host states (a STATE_DTYPE array, e.g. from rkv_state_init_host)
    by `steps` steps in place, as that many rkv_advance calls would."""
    if states.dtype != STATE_DTYPE or not states.flags.c_contiguous or \
            states.shape != (cfg.num_streams,):
        raise ValueError("states must be a contiguous STATE_DTYPE array of num_streams entries")
    _check("rkv_state_advance_host",
           lib().rkv_state_advance_host(ctypes.byref(cfg), states.ctypes.data, int(steps)))
    return states


def rkv_reset_streams(cfg, state, plan, streams, origin, stream=None):
    """Restart the decoder caches of `streams` at positions `origin` (host
    sequences); `plan`: None, or the already written plan of the coming step
    (pipelined loops), whose entries for these streams are rewritten."""
    st = np.ascontiguousarray(np.asarray(streams, dtype=np.int32).reshape(-1))
    org = np.ascontiguousarray(np.broadcast_to(np.asarray(origin, dtype=np.int64), st.shape))
    _check("rkv_reset_streams",
           lib().rkv_reset_streams(ctypes.byref(cfg), _ptr(state), _ptr(plan), int(st.size),
                                   st.ctypes.data if st.size else None,
                                   org.ctypes.data if st.size else None, _stream(stream)))


def make_restart_cfg(max_decode_kv=RKV_STREAM_MAX_DECODE_KV, eos_token=-1, text_token_min=0,
                     nontext_run=0, stall_steps=0) -> rkv_restart_cfg:
    return rkv_restart_cfg(max_decode_kv, eos_token, text_token_min, nontext_run, stall_steps)


def rkv_restart_step(cfg, state, tokens):
    """One clock step of the continuous-mode restart policy (host only).
    state: RESTART_STATE_DTYPE array of S entries, updated in place; tokens:
    the S tokens emitted this step (< 0: none).  Returns (streams to restart,
    per-stream reasons)."""
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
    if state.dtype != RESTART_STATE_DTYPE or not state.flags.c_contiguous or state.size != tok.size:
        raise ValueError("state must be a contiguous RESTART_STATE_DTYPE array, one entry per token")
    reason = np.zeros(tok.size, np.int32)
    restart = np.zeros(tok.size, np.int32)
    n = lib().rkv_restart_step(ctypes.byref(cfg), state.ctypes.data, int(tok.size),
                               tok.ctypes.data, reason.ctypes.data, restart.ctypes.data)
    if n < 0:
        raise RkvError("rkv_restart_step", n)
    return restart[:n].copy(), reason


def make_encoder_cfg(ffn=5120, norm_eps=1e-5) -> rkv_encoder_cfg:
    return rkv_encoder_cfg(ffn, norm_eps, (ctypes.c_int32 * 2)(0, 0))


ENCODER_WEIGHT_ORDER = ("g1", "wq", "wk", "wv", "wo", "g2", "w1", "w2")


def pack_encoder_weights(layers):
    """Per-layer dicts of bfloat16 tensors -> one contiguous bfloat16 tensor in
    the library's layer layout (include/rkv.h, rkv_encoder_layer_weight_bytes)."""
    import torch
    return torch.cat([lw[n].reshape(-1) for lw in layers for n in ENCODER_WEIGHT_ORDER])


def rkv_encoder_layer_weight_bytes(cfg, ecfg) -> int:
    return int(lib().rkv_encoder_layer_weight_bytes(ctypes.byref(cfg), ctypes.byref(ecfg)))


def rkv_encoder_step_workspace_bytes(cfg, ecfg, slots) -> int:
    return int(lib().rkv_encoder_step_workspace_bytes(ctypes.byref(cfg), ctypes.byref(ecfg),
                                                      int(slots)))


def rkv_encoder_step(cfg, ecfg, plan, kv, weights, x, workspace, stream=None):
    nbytes = workspace.numel() * workspace.element_size()
    _check("rkv_encoder_step",
           lib().rkv_encoder_step(ctypes.byref(cfg), ctypes.byref(ecfg), _ptr(plan),
                                  ctypes.byref(kv), _ptr(weights), _ptr(x), _ptr(workspace),
                                  nbytes, _stream(stream)))


def make_tcond_cfg(num_layers, hidden, dim=256, num_conds=1, max_frame_len=8) -> rkv_tcond_cfg:
    return rkv_tcond_cfg(num_layers, hidden, dim, num_conds, max_frame_len,
                         (ctypes.c_int32 * 3)(0, 0, 0))


def rkv_tcond_delay_tokens(target_delay_ms, clock_ms):
    """(num_delay_tokens, frame_len) for a delay and an audio clock (host)."""
    n, f = ctypes.c_int32(), ctypes.c_int32()
    _check("rkv_tcond_delay_tokens",
           lib().rkv_tcond_delay_tokens(int(target_delay_ms), int(clock_ms), ctypes.byref(n),
                                        ctypes.byref(f)))
    return n.value, f.value


def rkv_tcond_prepare(tc, num_delay, frame_len, table, weights, mod, stream=None):
    """num_delay, frame_len: host sequences of tc.num_conds ints; table, weights:
    bfloat16 device tensors; mod: float32 [L, C, 2, hidden] device tensor."""
    n = np.ascontiguousarray(num_delay, dtype=np.int32)
    f = np.ascontiguousarray(frame_len, dtype=np.int32)
    if n.size != tc.num_conds or f.size != tc.num_conds:
        raise ValueError("one delay count and frame_len per condition")
    _check("rkv_tcond_prepare",
           lib().rkv_tcond_prepare(ctypes.byref(tc), n.ctypes.data, f.ctypes.data, _ptr(table),
                                   _ptr(weights), _ptr(mod), _stream(stream)))


def rkv_tcond_modulate(cfg, tc, mod, stream_cond, out, stream=None):
    _check("rkv_tcond_modulate",
           lib().rkv_tcond_modulate(ctypes.byref(cfg), ctypes.byref(tc), _ptr(mod),
                                    _ptr(stream_cond), _ptr(out), _stream(stream)))


def make_mel_cfg(num_streams, n_fft=400, hop=160, n_mels=128,
                 samples_per_step=1280) -> rkv_mel_cfg:
    return rkv_mel_cfg(num_streams, n_fft, hop, n_mels, samples_per_step, 0)


def rkv_mel_filters_host(cfg, sample_rate=16000.0) -> np.ndarray:
    """[n_mels, n_fft // 2 + 1] float32 mel filterbank (host)."""
    out = np.zeros((cfg.n_mels, cfg.n_fft // 2 + 1), np.float32)
    _check("rkv_mel_filters_host",
           lib().rkv_mel_filters_host(ctypes.byref(cfg), float(sample_rate), out.ctypes.data))
    return out


def rkv_mel_step(cfg, tail_in, tail_out, samples, filters, out, stream=None):
    _check("rkv_mel_step", lib().rkv_mel_step(ctypes.byref(cfg), _ptr(tail_in), _ptr(tail_out),
                                              _ptr(samples), _ptr(filters), _ptr(out),
                                              _stream(stream)))


class MelFrontend:
    """Device buffers of the rolling log-mel front end: two alternating sample
    tails (zero: every stream starts after n_fft - hop silent samples) and the
    filterbank."""

    def __init__(self, cfg, sample_rate=16000.0, device="cuda", filters=None):
        """filters: a host float32 [n_mels, n_fft // 2 + 1] filterbank to upload
        instead of the library's (rkv_mel_filters_host)."""
        import torch
        self.cfg = cfg
        keep = cfg.n_fft - cfg.hop
        self.tails = [torch.zeros((cfg.num_streams, keep), dtype=torch.float32, device=device)
                      for _ in range(2)]
        if filters is None:
            filters = rkv_mel_filters_host(cfg, sample_rate)
        filters = np.ascontiguousarray(filters, dtype=np.float32)
        if filters.shape != (cfg.n_mels, cfg.n_fft // 2 + 1):
            raise ValueError("filterbank must be [n_mels, n_fft // 2 + 1]")
        self.filters = torch.from_numpy(filters).to(device)
        self.parity = 0

    def step(self, samples, out, stream=None):
        """samples [S, samples_per_step] -> out [S, samples_per_step // hop, n_mels]."""
        a, b = self.tails[self.parity], self.tails[1 - self.parity]
        rkv_mel_step(self.cfg, a, b, samples, self.filters, out, stream)
        self.parity = 1 - self.parity


def rkv_workspace_bytes(cfg, slots) -> int:
    return int(lib().rkv_workspace_bytes(ctypes.byref(cfg), int(slots)))


def rkv_advance(cfg, state, plan, stream=None):
    _check("rkv_advance", lib().rkv_advance(ctypes.byref(cfg), _ptr(state), _ptr(plan),
                                            _stream(stream)))


def rkv_update_step(cfg, plan, kv, k_new, v_new, stream=None):
    _check("rkv_update_step", lib().rkv_update_step(ctypes.byref(cfg), _ptr(plan), ctypes.byref(kv),
                                                    _ptr(k_new), _ptr(v_new), _stream(stream)))


def rkv_append(cfg, plan, kv, k_new, v_new, stream=None):
    _check("rkv_append", lib().rkv_append(ctypes.byref(cfg), _ptr(plan), ctypes.byref(kv),
                                          _ptr(k_new), _ptr(v_new), _stream(stream)))


def rkv_roll_rebase(cfg, plan, kv, stream=None):
    _check("rkv_roll_rebase", lib().rkv_roll_rebase(ctypes.byref(cfg), _ptr(plan),
                                                    ctypes.byref(kv), _stream(stream)))


def rkv_compact(cfg, plan, kv, stream=None):
    _check("rkv_compact", lib().rkv_compact(ctypes.byref(cfg), _ptr(plan), ctypes.byref(kv),
                                            _stream(stream)))


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def rkv_decode_attn(cfg, plan, kv, q, out, workspace=None, stream=None):
    wp, wb = _ws(workspace)
    _check("rkv_decode_attn", lib().rkv_decode_attn(ctypes.byref(cfg), _ptr(plan),
                                                    ctypes.byref(kv), _ptr(q), _ptr(out),
                                                    wp, wb, _stream(stream)))


def rkv_decode_step(cfg, plan, kv, q, k_new, v_new, out, workspace=None, stream=None):
    wp, wb = _ws(workspace)
    _check("rkv_decode_step", lib().rkv_decode_step(ctypes.byref(cfg), _ptr(plan),
                                                    ctypes.byref(kv), _ptr(q), _ptr(k_new),
                                                    _ptr(v_new), _ptr(out), wp, wb,
                                                    _stream(stream)))


def rkv_decode_step_noalloc(cfg, plan, kv, q, k_new, v_new, out, stream=None):
    """rkv_decode_step with the library's own split-partial array instead of a
    workspace (no allocation)."""
    _check("rkv_decode_step_noalloc",
           lib().rkv_decode_step_noalloc(ctypes.byref(cfg), _ptr(plan), ctypes.byref(kv),
                                         _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out),
                                         _stream(stream)))


def rkv_decode_attn_pipelined(cfg, state, plan, plan_next, kv, q, out, workspace=None,
                              stream=None):
    """rkv_decode_attn with `plan`, and the next step's plan into `plan_next`
    (state advanced) in the same launch."""
    wp, wb = _ws(workspace)
    _check("rkv_decode_attn_pipelined",
           lib().rkv_decode_attn_pipelined(ctypes.byref(cfg), _ptr(state), _ptr(plan),
                                           _ptr(plan_next), ctypes.byref(kv), _ptr(q), _ptr(out),
                                           wp, wb, _stream(stream)))


def rkv_decode_step_pipelined(cfg, state, plan, plan_next, kv, q, k_new, v_new, out,
                              workspace=None, stream=None):
    """rkv_decode_step with `plan`, and the next step's plan into `plan_next`
    (state advanced) in the same launch."""
    wp, wb = _ws(workspace)
    _check("rkv_decode_step_pipelined",
           lib().rkv_decode_step_pipelined(ctypes.byref(cfg), _ptr(state), _ptr(plan),
                                           _ptr(plan_next), ctypes.byref(kv), _ptr(q),
                                           _ptr(k_new), _ptr(v_new), _ptr(out), wp, wb,
                                           _stream(stream)))


def rkv_decode_step_pipelined_tcond(cfg, tc, mod, stream_cond, state, plan, plan_next, kv, q,
                                    k_new, v_new, out, workspace=None, stream=None):
    """rkv_decode_step_pipelined with the delay conditioning of
    rkv_tcond_modulate applied as the output is stored (same bits)."""
    wp, wb = _ws(workspace)
    _check("rkv_decode_step_pipelined_tcond",
           lib().rkv_decode_step_pipelined_tcond(ctypes.byref(cfg), ctypes.byref(tc), _ptr(mod),
                                                 _ptr(stream_cond), _ptr(state), _ptr(plan),
                                                 _ptr(plan_next), ctypes.byref(kv), _ptr(q),
                                                 _ptr(k_new), _ptr(v_new), _ptr(out), wp, wb,
                                                 _stream(stream)))


def rkv_encoder_chunk_attn(cfg, plan, kv, q, k_new, v_new, out, workspace=None, stream=None):
    wp, wb = _ws(workspace)
    _check("rkv_encoder_chunk_attn",
           lib().rkv_encoder_chunk_attn(ctypes.byref(cfg), _ptr(plan), ctypes.byref(kv), _ptr(q),
                                        _ptr(k_new), _ptr(v_new), _ptr(out), wp, wb,
                                        _stream(stream)))


# ---------------------------------------------------------------------------
# device buffers for one cache (torch is only the allocator)
# ---------------------------------------------------------------------------

class Cache:
    """Device tensors of one rolling cache: rings, per-stream state, plan, workspace.

    layout "interleaved" (default): one buffer [L, S, Hkv, slots, n, d] with K,
    V (and the compensated residual) of a slot side by side, so a slot's rows
    are one contiguous stream; "separate": three [L, S, Hkv, slots, d] tensors.
    Either is described to the library through strides (rkv_kv_view).
    """

    def __init__(self, cfg, slots, window, cap, origin=0, device="cuda", zero=True,
                 layout="interleaved"):
        import torch
        if cfg.max_cap == 0:
            cfg.max_cap = slots      # the rings below hold `slots` rows per head
        self.cfg = cfg
        L, S, H, d = cfg.num_layers, cfg.num_streams, cfg.num_kv_heads, cfg.head_dim
        comp = bool(cfg.flags & RKV_F_COMPENSATED)
        # storage format of K, V, k_lo: bfloat16, or binary16 (RKV_F_KV_FP16)
        dt = torch.float16 if cfg.flags & RKV_F_KV_FP16 else torch.bfloat16
        alloc = torch.zeros if zero else torch.empty
        if layout == "interleaved":
            n = 3 if comp else 2
            self.buf = alloc((L, S, H, slots, n, d), dtype=dt, device=device)
            self.k = self.buf[:, :, :, :, 0, :]
            self.v = self.buf[:, :, :, :, 1, :]
            self.k_lo = self.buf[:, :, :, :, 2, :] if comp else None
        elif layout == "separate":
            shape = (L, S, H, slots, d)
            self.k = alloc(shape, dtype=dt, device=device)
            self.v = alloc(shape, dtype=dt, device=device)
            self.k_lo = alloc(shape, dtype=dt, device=device) if comp else None
        else:
            raise ValueError(layout)
        self.kv = kv_view(self.k, self.v, self.k_lo)
        self.state = torch.empty(cfg.num_streams * STATE_DTYPE.itemsize, dtype=torch.uint8,
                                 device=device)
        with torch.cuda.device(self.state.device):
            rkv_state_init(cfg, self.state, window, cap, origin)
        self.plan = torch.zeros(S * PLAN_DTYPE.itemsize, dtype=torch.uint8, device=device)
        # second plan buffer for rkv_decode_step_pipelined (plans alternate)
        self.plan_next = torch.zeros_like(self.plan)
        nbytes = rkv_workspace_bytes(cfg, slots)
        # zero-filled: the merge counters at its start must be zero at the first call
        self.workspace = (torch.zeros((nbytes + 3) // 4, dtype=torch.float32, device=device)
                          if nbytes else None)

    def plan_host(self) -> np.ndarray:
        return self.plan.cpu().numpy().view(PLAN_DTYPE)

    def state_host(self) -> np.ndarray:
        return self.state.cpu().numpy().view(STATE_DTYPE)


def default_scale(d):
    return 1.0 / math.sqrt(d)
