// Per-stream step plan (device code shared by the plan kernel and the
// pipelined decode step, so both write identical plans).
//
// REBASE  (Audio8 explainer, "Rolling KV Cache 三步拆解" steps 1-2): the ring
//   holds the last W tokens; when full the oldest is pushed out and its slot
//   reused.  The base b moves in multiples of the re-base chunk: b is the
//   largest multiple not above the oldest retained position, and when it moves
//   by D the retained K are rotated by R(-D).  The new token is written at
//   relative position t - b.
// COMPACT (voxtral.c explainer, section 二): rows grow to the capacity; when
//   full, the newest W rows are kept (moved to row 0 by rkv_compact) and
//   kv_pos_offset grows by the number dropped; the new row's rotary position
//   is kv_pos_offset + its row.
// ENC_CHUNK (same explainer, section 三): F frames per step into a ring of
//   cap >= W + F slots at logical positions; frames attend back to
//   max(origin, P - W).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "rkv.h"

namespace rkv {

// theta_i = base^(-2i/d) for i < d/2, computed once on the host in float64.
struct Theta {
  double v[RKV_MAX_HEAD_DIM / 2];
};

struct PlanHead {
  int64_t t, pos, pos_offset, first_pos, evict_pos;
  int32_t slot, n_valid, delta, drop, evict_slot, new_rows;
  rkv_stream_state next;
};

// State before the first step of a stream whose first position is `origin`
// (window and capacity already validated for the mode).
__host__ __device__ inline rkv_stream_state initial_state(int64_t origin, int32_t window,
                                                          int32_t cap, int mode, int dc) {
  rkv_stream_state st;
  st.t = origin - 1;
  st.origin = origin;
  st.pos_offset = mode == RKV_MODE_REBASE ? (int64_t)dc * (origin / dc) : origin;
  st.len = 0;
  st.window = window;
  st.cap = cap;
  st.reserved[0] = st.reserved[1] = st.reserved[2] = 0;
  return st;
}

// One step's plan header and the state after it (host and device: the host
// uses it to advance states without launches).
__host__ __device__ inline PlanHead make_plan(const rkv_stream_state& x, int mode, int dc,
                                              int F) {
  PlanHead p;
  p.next = x;
  p.delta = 0;
  p.drop = 0;
  p.evict_pos = -1;
  p.evict_slot = -1;
  p.new_rows = 1;
  if (mode == RKV_MODE_REBASE) {
    const int64_t t = x.t + 1;
    int32_t len = x.len;
    if (len == x.window) {
      p.evict_pos = t - x.window;
      p.evict_slot = (int32_t)((t - x.origin) % x.window);
    } else {
      len += 1;
    }
    const int64_t oldest = t - len + 1;
    const int64_t base = (int64_t)dc * (oldest / dc);
    p.t = t;
    p.slot = (int32_t)((t - x.origin) % x.window);
    p.n_valid = len;
    p.delta = (int32_t)(base - x.pos_offset);
    p.pos = t - base;
    p.pos_offset = base;
    p.first_pos = oldest;
    p.next.t = t;
    p.next.len = len;
    p.next.pos_offset = base;
  } else if (mode == RKV_MODE_COMPACT) {
    const int64_t t = x.t + 1;
    int32_t len = x.len;
    int64_t off = x.pos_offset;
    if (len >= x.cap && len >= x.window) {
      p.drop = len - x.window;
      p.evict_pos = off;
      off += p.drop;
      len = x.window;
    }
    p.t = t;
    p.slot = len;
    len += 1;
    p.n_valid = len;
    p.pos = off + p.slot;
    p.pos_offset = off;
    p.first_pos = off;
    p.next.t = t;
    p.next.len = len;
    p.next.pos_offset = off;
  } else {  // RKV_MODE_ENC_CHUNK
    const int64_t first = x.t + 1;
    p.t = x.t + F;
    p.slot = (int32_t)((first - x.origin) % x.cap);
    const int32_t len = x.len + F < x.cap ? x.len + F : x.cap;
    p.n_valid = len;
    p.pos = first;
    p.pos_offset = x.origin;
    p.first_pos = first - x.window > x.origin ? first - x.window : x.origin;
    p.new_rows = F;
    p.next.t = p.t;
    p.next.len = len;
  }
  return p;
}

// Advance stream s by one step from state x with the 64 lanes of one wave
// (lane = 0..63; every lane holds x): lane 0 publishes the plan header and the
// new state; lane i < d/2 fills the rotary tables of pair i, only for the
// rows and pairs a step uses (rows j < new_rows; a zero delta has the exact
// table cos = 1, sin = 0).
__device__ inline void advance_from(const rkv_stream_state& x, rkv_stream_state* __restrict__ st,
                                    rkv_step_plan* __restrict__ plan, int s, int lane, int mode,
                                    int dc, int F, int half, const Theta& th) {
  const PlanHead p = make_plan(x, mode, dc, F);
  rkv_step_plan* out = plan + s;
  if (lane == 0) {
    st[s] = p.next;
    out->t = p.t;
    out->pos = p.pos;
    out->pos_offset = p.pos_offset;
    out->first_pos = p.first_pos;
    out->evict_pos = p.evict_pos;
    out->slot = p.slot;
    out->n_valid = p.n_valid;
    out->rebase_delta = p.delta;
    out->compact_drop = p.drop;
    out->evict_slot = p.evict_slot;
    out->window = x.window;
    out->cap = x.cap;
    out->new_rows = p.new_rows;
    for (int r = 0; r < 14; ++r) out->reserved[r] = 0;
  }
  if (lane >= half) return;
  const double theta = th.v[lane];
#pragma unroll 1
  for (int j = 0; j < p.new_rows; ++j) {
    double sn, cs;
    sincos((double)(p.pos + j) * theta, &sn, &cs);
    out->rope_new[j][0][lane] = cs;
    out->rope_new[j][1][lane] = sn;
  }
  double sn = 0.0, cs = 1.0;
  if (p.delta != 0) sincos((double)p.delta * theta, &sn, &cs);
  out->rope_delta[0][lane] = cs;
  out->rope_delta[1][lane] = sn;
}

// Advance stream s by one step from its stored state: every lane reads the
// old state first (the loads of one wave complete before any of its later
// stores, so lane 0 may then overwrite it).
__device__ inline void advance_stream(rkv_stream_state* __restrict__ st,
                                      rkv_step_plan* __restrict__ plan, int s, int lane, int mode,
                                      int dc, int F, int half, const Theta& th) {
  const rkv_stream_state x = st[s];
  advance_from(x, st, plan, s, lane, mode, dc, F, half, th);
}

// Host: the theta table of a configuration.
inline Theta theta_table(const rkv_cfg* cfg) {
  Theta th;
  const int half = cfg->head_dim / 2;
  for (int i = 0; i < RKV_MAX_HEAD_DIM / 2; ++i)
    th.v[i] = i < half ? pow(cfg->rope_base, -2.0 * (double)i / (double)cfg->head_dim) : 0.0;
  return th;
}

}  // namespace rkv
