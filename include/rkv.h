/*
 * rkv.h -- rolling-window KV cache for streaming decode on AMD gfx950 (C ABI).
 *
 * The library computes one clock step of the streaming decoder's attention
 * over a bounded KV cache, for a batch of independent streams and a range of
 * layers, entirely in hand-written HIP kernels.  The three cache disciplines
 * follow the pages this library implements:
 *
 *   RKV_MODE_REBASE  -- "Audio8 ASR Infinite" explainer (m.lsln.cn), section
 *       "Rolling KV Cache 三步拆解": a fixed ~30 s window (W positions), the
 *       oldest token pushed out per step, and exact RoPE re-basing: retained K
 *       are rotated in place by R(-D) when the position base moves by D, so
 *       stored positions stay inside the window.  Also the model card
 *       (Edge0/Audio8-ASR-Infinite), "使用 vLLM 进行全天候推理".
 *   RKV_MODE_COMPACT -- voxtral.c rolling-KV explainer (kwkr.cn), section 二:
 *       the buffer grows to its capacity, then the newest W rows move to row 0
 *       and the dropped count is added to kv_pos_offset; the rotary position
 *       of a row is kv_pos_offset + its physical index, and K is never
 *       rewritten.
 *   RKV_MODE_ENC_CHUNK -- same explainer, section 三: the encoder appends a
 *       chunk of F frames per step and attends to a 750-frame window of cached
 *       K/V; here the window is a ring of W + F slots at logical positions.
 *
 * Conventions
 *   - Every entry point returns 0 (RKV_OK) or a negative rkv_status.  All
 *     arguments are validated on the host before any HIP call, so errors are
 *     reported without touching a device.  No exception or abort crosses the
 *     ABI.
 *   - Device pointers are plain HIP device addresses; the caller allocates
 *     and frees every buffer (rings, state, plan, inputs, outputs, workspace).
 *     The library allocates no memory and keeps no global state besides the
 *     thread-local last HIP error, so calls on different HIP streams with
 *     disjoint buffers may run concurrently.
 *   - Calls are asynchronous on the given hipStream_t (passed as void*; NULL
 *     is the default stream).  Calls that share buffers must be ordered by
 *     the caller (one stream does that).
 *   - Element type of K, V, q, k_new, v_new is bfloat16 (raw 16-bit patterns).
 *     Output is bfloat16, or float32 with RKV_F_OUT_F32.
 *   - Rotary embedding: theta_i = rope_base^(-2i/d), i < d/2; element i pairs
 *     with element i + d/2 (half-split).  Angles and their cosines/sines are
 *     float64.  An appended K (rkv_append and the appends inside the fused
 *     calls) is rotated in float64 and stored as the correctly rounded
 *     (nearest, ties to even) value.  A re-base of stored K (rkv_roll_rebase
 *     and the re-bases inside the fused calls) is rotated in float32
 *     double-float arithmetic (cos/sin split into float32 hi + lo, product
 *     errors recovered with FMAs) and rounded to nearest: within 1 ulp of the
 *     correctly rounded float64 rotation.
 *   - Capacity: rkv_cfg.max_cap declares the rows per (layer, stream, head)
 *     the caller's rings hold.  rkv_state_init rejects a stream capacity above
 *     it and every call that takes an rkv_kv_view rejects kv->slots below it
 *     (RKV_ESTATE), so no stream state can address a row the ring lacks.
 */
#ifndef RKV_H
#define RKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RKV_VERSION 1
#define RKV_MAX_HEAD_DIM 128
#define RKV_MAX_NEW_ROWS 8   /* frames per encoder chunk */
#define RKV_MAX_GROUP 8      /* query vectors sharing one KV head */

typedef enum rkv_status {
  RKV_OK = 0,
  RKV_EINVAL = -1,       /* null pointer, non-positive size, inconsistent sizes */
  RKV_EUNSUPPORTED = -2, /* head_dim not 64/128, group > 8, F > 8, unknown mode/flag */
  RKV_EALIGN = -3,       /* pointer not 16-byte aligned or stride not a multiple of 8 elements */
  RKV_ESTATE = -4,       /* per-stream window/capacity/origin inconsistent with the mode,
                            or a ring with fewer slots than cfg->max_cap */
  RKV_EHIP = -5,         /* a HIP launch failed; see rkv_last_hip_error() */
  RKV_ESPACE = -6        /* workspace smaller than rkv_workspace_bytes() */
} rkv_status;

typedef enum rkv_mode {
  RKV_MODE_REBASE = 0,
  RKV_MODE_COMPACT = 1,
  RKV_MODE_ENC_CHUNK = 2
} rkv_mode;

enum {
  /* REBASE mode: keep the bfloat16 rounding residual of every K in kv->k_lo
   * and re-base the pair hi + lo, so repeated re-bases do not accumulate
   * rounding (needed when the base moves every step).  Attention reads hi. */
  RKV_F_COMPENSATED = 1u << 0,
  /* write attention output as float32 instead of bfloat16 */
  RKV_F_OUT_F32 = 1u << 1,
  /* fp16 cache variant (voxtral.c explainer, section 七, "fp16 KV cache"):
   * K, V and k_lo are stored as IEEE binary16 (11 significant bits; every
   * stored value rounded to nearest, ties to even, from the float64 rotation
   * or, for V, from the bfloat16 input); q, k_new, v_new stay bfloat16 and
   * the matrix-core products run in fp16.  REBASE and COMPACT modes only
   * (RKV_EUNSUPPORTED for ENC_CHUNK). */
  RKV_F_KV_FP16 = 1u << 2,
  /* When a call splits the key range (rkv_workspace_bytes() > 0), always
   * merge the splits' partial results in a second launch (same results, bit
   * for bit).  Without it, a split launch of at most 768 workgroups (items x
   * splits: one round on the chip) merges in the attention launch itself --
   * the last split of each (layer, stream, head) to finish merges, counted by
   * per-item counters in the workspace, which must then be zero at the first
   * call -- and larger ones in a second launch. */
  RKV_F_MERGE_LAUNCH = 1u << 3
};

/* Problem description, shared by every call of a step (host memory). */
typedef struct rkv_cfg {
  int32_t num_streams;   /* S >= 1 */
  int32_t num_layers;    /* L >= 1 layers handled by one call */
  int32_t num_q_heads;   /* Hq; ENC_CHUNK: heads H (multi-head, Hq == Hkv) */
  int32_t num_kv_heads;  /* Hkv; Hq / Hkv <= 8 */
  int32_t head_dim;      /* d: 64 or 128 */
  int32_t mode;          /* rkv_mode */
  int32_t rebase_chunk;  /* REBASE: the base moves in multiples of this (>= 1) */
  int32_t new_rows;      /* rows appended per step: 1, or F (1..8) for ENC_CHUNK */
  uint32_t flags;        /* RKV_F_* */
  int32_t num_splits;    /* key-range splits per (layer, stream, head), at most 64 and one
                            per 16 slots are used; 0 = library choice */
  double rope_base;      /* > 0, e.g. 1e6 */
  float softmax_scale;   /* 0 = 1/sqrt(d) */
  int32_t max_cap;       /* rows per (layer, stream, head) of the rings: >= every stream's
                            capacity and <= kv->slots (RKV_ESTATE otherwise); >= 1 for
                            rkv_state_init* and every call taking an rkv_kv_view
                            (RKV_EINVAL otherwise), unused by the others */
} rkv_cfg;

/* Per-stream cache state (device memory, S entries, 48 bytes each).
 * Built by rkv_state_init (or rkv_state_init_host and a copy by the caller);
 * afterwards only rkv_advance writes it. */
typedef struct rkv_stream_state {
  int64_t t;          /* REBASE/COMPACT: step of the last appended token;
                         ENC_CHUNK: position of the last appended frame; origin-1 at start */
  int64_t origin;     /* first position of the stream */
  int64_t pos_offset; /* REBASE: base b; COMPACT: kv_pos_offset; ENC_CHUNK: origin */
  int32_t len;        /* valid rows */
  int32_t window;     /* W */
  int32_t cap;        /* ring slots used by this stream (<= kv->slots) */
  int32_t reserved[3];
} rkv_stream_state;

/* Per-stream plan of the current step (device memory, S entries), written by
 * rkv_advance and read by every other call of the step. */
typedef struct rkv_step_plan {
  int64_t t;            /* step (frame position of the last new frame for ENC_CHUNK) */
  int64_t pos;          /* rotary position of the first new row: t - base (REBASE),
                           kv_pos_offset + slot (COMPACT), frame position (ENC_CHUNK) */
  int64_t pos_offset;   /* base / kv_pos_offset / origin after this step */
  int64_t first_pos;    /* oldest position the new row(s) attend to */
  int64_t evict_pos;    /* REBASE: position pushed out; COMPACT: first dropped; -1 none */
  int32_t slot;         /* physical slot of the first new row */
  int32_t n_valid;      /* rows valid (attended) after the append */
  int32_t rebase_delta; /* D: retained K rotate by R(-D) before the append; 0 none */
  int32_t compact_drop; /* rows dropped by this step's compaction; 0 none */
  int32_t evict_slot;   /* REBASE: slot of the pushed-out token; -1 none */
  int32_t window;
  int32_t cap;
  int32_t new_rows;
  int32_t reserved[14];
  double rope_new[RKV_MAX_NEW_ROWS][2][RKV_MAX_HEAD_DIM / 2]; /* cos, sin of (pos + j) theta_i;
                                                                written for j < new_rows, i < d/2 */
  double rope_delta[2][RKV_MAX_HEAD_DIM / 2];                 /* cos, sin of D theta_i, i < d/2 */
} rkv_step_plan;

/* Where the cache lives (host struct describing device memory).
 * Element (layer l, stream s, kv head g, slot r, e) of K is at
 *   k + l*layer_stride + s*stream_stride + g*head_stride + r*slot_stride + e
 * (strides in bfloat16 elements); V and k_lo use the same strides.
 * The canonical layout is [L][S][Hkv][slots][d] with slot_stride = d. */
typedef struct rkv_kv_view {
  void* k;
  void* v;
  void* k_lo;             /* RKV_F_COMPENSATED only, else may be NULL */
  int64_t layer_stride;
  int64_t stream_stride;
  int64_t head_stride;
  int64_t slot_stride;    /* >= d */
  int32_t slots;          /* rows allocated per (layer, stream, head) */
  int32_t reserved;
} rkv_kv_view;

/* Library version (RKV_VERSION). */
int rkv_version(void);

/* Static description of a status code (never NULL). */
const char* rkv_strerror(int status);

/* hipError_t of the last RKV_EHIP returned on the calling thread (0 if none). */
int rkv_last_hip_error(void);

/* Check a configuration without touching a device. */
int rkv_validate_cfg(const rkv_cfg* cfg);

/* Fill h_state[0..S) (host memory) for streams starting at h_origin[s] with
 * window h_window[s] and capacity h_cap[s].  Required: REBASE cap == window;
 * COMPACT cap > window (the voxtral.c window plus room to grow before the next
 * compaction); ENC_CHUNK cap >= window + new_rows; cap <= cfg->max_cap;
 * origin >= 0 (RKV_ESTATE otherwise; RKV_EINVAL for max_cap < 1).  The caller
 * copies the array to device memory (S * sizeof(rkv_stream_state) bytes). */
int rkv_state_init_host(const rkv_cfg* cfg, const int32_t* h_window,
                        const int32_t* h_cap, const int64_t* h_origin,
                        rkv_stream_state* h_state);

/* Host: advance h_state[0..S) by `steps` steps in place, with exactly the
 * state changes of `steps` rkv_advance calls (the step rules of the three
 * modes: Audio8 explainer "Rolling KV Cache 三步拆解" steps 1-2, voxtral.c
 * explainer sections 二 and 三), without writing plans or touching a device.
 * For callers that resume streams at a known step without replaying the
 * launches (rings filled by other means, checkpoints).  The states must be
 * ones the rules can reach from rkv_state_init_host: window >= 1, 0 <= len <=
 * cap <= cfg->max_cap, origin >= 0, t >= origin - 1 and the mode's capacity
 * rule (RKV_ESTATE otherwise); steps >= 0 and max_cap >= 1 (RKV_EINVAL).  On
 * an error no state is changed. */
int rkv_state_advance_host(const rkv_cfg* cfg, rkv_stream_state* h_state, int64_t steps);

/* The same initial states as rkv_state_init_host, written to d_state[0..S)
 * (device memory, 8-byte aligned) with copies on hip_stream.  Host arrays as
 * above.  Blocks until the copies are done (set-up, not the per-step path);
 * validation errors return before any HIP call, RKV_EHIP if a copy fails.
 * Per-stream window, capacity and start: the mixed-clock pool of the Audio8
 * model card (streams of different clocks in one batch). */
int rkv_state_init(const rkv_cfg* cfg, rkv_stream_state* d_state, const int32_t* h_window,
                   const int32_t* h_cap, const int64_t* h_origin, void* hip_stream);

/* Bytes of workspace rkv_decode_attn / rkv_decode_step /
 * rkv_encoder_chunk_attn need for a cache of `slots` rows per head (0 when
 * the key range is not split).  Layout: one uint32 merge counter per
 * (layer, stream, kv head) item, padded to 256 bytes, then the float32 split
 * partials.  Unless cfg has RKV_F_MERGE_LAUNCH the counters must be zero when
 * a call starts: zero-fill a new workspace before its first use (and after
 * using it with another configuration); every call leaves them zero when its
 * launch completes. */
size_t rkv_workspace_bytes(const rkv_cfg* cfg, int32_t slots);

/* Step plan (Audio8 explainer "Rolling KV Cache 三步拆解" steps 1-2; voxtral.c
 * explainer section 二 trigger and logical position; section 三 encoder chunk):
 * advance every stream by one step, update d_state in place and write
 * d_plan[S] including the rotary cos/sin tables for the new row(s) and for
 * the re-base angle.  Once per clock step, shared by all layers. */
int rkv_advance(const rkv_cfg* cfg, rkv_stream_state* d_state,
                rkv_step_plan* d_plan, void* hip_stream);

/* Fused RoPE-on-append (voxtral.c explainer section 二: the rotation is baked
 * into K when it is written).  For each (layer, stream, kv head) and new row
 * j: K[slot_j] = rne(R(pos + j) k_new), V[slot_j] = v_new (and, compensated,
 * k_lo[slot_j] = rne(R(pos + j) k_new - K[slot_j])), slot_j = (slot + j) mod cap.
 * k_new, v_new: bfloat16 [L][S][Hkv][d] (ENC_CHUNK: [L][S][F][H][d]). */
int rkv_append(const rkv_cfg* cfg, const rkv_step_plan* d_plan,
               const rkv_kv_view* kv, const void* k_new, const void* v_new,
               void* hip_stream);

/* Exact re-base (Audio8 explainer "Rolling KV Cache 三步拆解" step 2): for
 * streams whose plan has rebase_delta D > 0, every retained K row (rows
 * [0, n_valid) except the new row's slot) becomes rne(R(-D) K) in place
 * (compensated: x = K + k_lo, K = rne(R(-D) x), k_lo = rne(R(-D) x - K)).
 * The rotation is an exact rotation matrix evaluated in float32 (cos/sin
 * rounded from the plan's float64 tables), each result rounded to nearest
 * bfloat16: within 1 ulp of the correctly rounded value, and bit-identical to
 * the re-base inside rkv_decode_step.
 * REBASE mode only; call after rkv_advance and before rkv_append. */
int rkv_roll_rebase(const rkv_cfg* cfg, const rkv_step_plan* d_plan,
                    const rkv_kv_view* kv, void* hip_stream);

/* The cache updates of one step in one launch: the re-base of rkv_roll_rebase
 * (for the streams whose base moves) and the append of rkv_append, with the
 * same ring contents as those two calls in that order (the re-base skips the
 * new row's slot, the append writes only it, so the two are independent).
 * Any mode (COMPACT and ENC_CHUNK plans never move the base; in COMPACT mode
 * call rkv_compact first).  Arguments and errors as rkv_append. */
int rkv_update_step(const rkv_cfg* cfg, const rkv_step_plan* d_plan,
                    const rkv_kv_view* kv, const void* k_new, const void* v_new,
                    void* hip_stream);

/* Compaction (voxtral.c explainer section 二): for streams whose plan has
 * compact_drop D > 0, move K and V rows [D, D + window) to [0, window) in
 * row order (an overlapping forward move, done in place).  COMPACT mode only;
 * call after rkv_advance and before rkv_append. */
int rkv_compact(const rkv_cfg* cfg, const rkv_step_plan* d_plan,
                const rkv_kv_view* kv, void* hip_stream);

/* GQA decode attention over the cache (Audio8 explainer "Rolling KV Cache
 * 三步拆解" step 3: attention scans only the fixed window).  For each layer,
 * stream and query head h (KV head h / (Hq/Hkv)): out = softmax(scale *
 * (R(pos) q_h) . K_r) V_r over rows r in [0, n_valid), with the query rotated
 * at the plan's position.  q, out: [L][S][Hq][d].  Reads the cache as stored
 * (call after rkv_append).  `workspace` may be NULL when
 * rkv_workspace_bytes() is 0. */
int rkv_decode_attn(const rkv_cfg* cfg, const rkv_step_plan* d_plan,
                    const rkv_kv_view* kv, const void* q, void* out,
                    void* workspace, size_t workspace_bytes, void* hip_stream);

/* One decoder step in a single pass over the cache: re-base (REBASE),
 * append, and decode attention, with results identical to rkv_roll_rebase +
 * rkv_append + rkv_decode_attn (COMPACT: rkv_compact must still run first). */
int rkv_decode_step(const rkv_cfg* cfg, const rkv_step_plan* d_plan,
                    const rkv_kv_view* kv, const void* q, const void* k_new,
                    const void* v_new, void* out, void* workspace,
                    size_t workspace_bytes, void* hip_stream);

/* rkv_decode_step for callers that cannot allocate device memory (code under
 * HIP graph capture, fixed serving loops, harnesses that forbid allocation):
 * the key-range split partials live in a device array of the library's own
 * (RKV_NOALLOC_SCRATCH_BYTES per GPU, held from the first call on a device
 * until the process ends) instead of a caller workspace; no allocation, same
 * kernels and the same results as rkv_decode_step.  The first call on a
 * device looks the array up (hipGetSymbolAddress, not a stream operation):
 * make one call before capturing a graph.  The current device must be the
 * one hip_stream belongs to.  Every call on a GPU shares that GPU's array
 * and leaves its contents behind; calls whose launches may overlap in time on
 * one GPU (unordered streams) race and give wrong results.  The array ends
 * in RKV_NOALLOC_MAX_SPLIT_ITEMS merge counters (zero at load; every call
 * leaves them zero), the rest holds the split partials.  Errors as
 * rkv_decode_step, and RKV_ESPACE when a split call's partials (the
 * workspace minus its counters) exceed the rest of the array or it has more
 * than RKV_NOALLOC_MAX_SPLIT_ITEMS items (checked before any HIP call). */
#define RKV_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
#define RKV_NOALLOC_MAX_SPLIT_ITEMS 16384 /* items of a split call; counters at the array's end */
int rkv_decode_step_noalloc(const rkv_cfg* cfg, const rkv_step_plan* d_plan,
                            const rkv_kv_view* kv, const void* q, const void* k_new,
                            const void* v_new, void* out, void* hip_stream);

/* Pipelined decode step for callers that keep two plan buffers: the decode
 * step of rkv_decode_step with d_plan, and in the same launch the next step's
 * plan written to d_plan_next with d_state advanced, exactly what
 * rkv_advance(d_state, d_plan_next) would write.  The sequence
 *   rkv_advance(state, A); pipelined(state, A, B); pipelined(state, B, A); ...
 * gives bit-identical rings, outputs, states and plans to rkv_advance +
 * rkv_decode_step per step, with one launch per step instead of two (the
 * plan of the Audio8 explainer's "Rolling KV Cache 三步拆解" steps 1-2 is
 * only needed by the next step).  d_plan and d_plan_next must not overlap
 * (RKV_EINVAL); d_state 8-byte and d_plan_next 16-byte aligned.  In
 * COMPACT mode call rkv_compact with d_plan first, as for rkv_decode_step. */
int rkv_decode_step_pipelined(const rkv_cfg* cfg, rkv_stream_state* d_state,
                              const rkv_step_plan* d_plan, rkv_step_plan* d_plan_next,
                              const rkv_kv_view* kv, const void* q, const void* k_new,
                              const void* v_new, void* out, void* workspace,
                              size_t workspace_bytes, void* hip_stream);

/* Pipelined read-only attention: rkv_decode_attn with d_plan, and in the same
 * launch the next step's plan written to d_plan_next with d_state advanced,
 * exactly as in rkv_decode_step_pipelined.  For the update path
 *   rkv_advance(state, A);
 *   rkv_update_step(A); attn_pipelined(state, A, B);
 *   rkv_update_step(B); attn_pipelined(state, B, A); ...
 * which gives the same rings, outputs, states and plans as rkv_advance +
 * rkv_update_step + rkv_decode_attn per step in two launches instead of
 * three.  REBASE and COMPACT modes (COMPACT: rkv_compact with the step's plan
 * before rkv_update_step); alignment and overlap rules as
 * rkv_decode_step_pipelined. */
int rkv_decode_attn_pipelined(const rkv_cfg* cfg, rkv_stream_state* d_state,
                              const rkv_step_plan* d_plan, rkv_step_plan* d_plan_next,
                              const rkv_kv_view* kv, const void* q, void* out,
                              void* workspace, size_t workspace_bytes, void* hip_stream);

/* Encoder chunk attention (voxtral.c explainer section 三: only the new
 * positions are computed, against the cached K/V of the window).  Appends the
 * F frames of the chunk (as rkv_append) and computes, for every head and frame
 * j, attention over the frames at positions [first_pos, pos + j] held in the
 * ring.  q, k_new, v_new, out: [L][S][F][H][d].  ENC_CHUNK mode only. */
int rkv_encoder_chunk_attn(const rkv_cfg* cfg, const rkv_step_plan* d_plan,
                           const rkv_kv_view* kv, const void* q,
                           const void* k_new, const void* v_new, void* out,
                           void* workspace, size_t workspace_bytes,
                           void* hip_stream);

/* ---------------------------------------------------------------------------
 * Continuous mode (voxtral.c explainer, section 四).  In live transcription
 * the decoder is restarted hard -- its context is dropped -- when the model
 * ends an utterance (EOS), when its cache would grow past
 * STREAM_MAX_DECODE_KV positions (bounding the attention cost), on a run of
 * control tokens, and when audio advances while it produces nothing; the
 * encoder cache (a separate state) and the streaming pipeline keep running.
 * rkv_restart_step decides on the host; rkv_reset_streams restarts caches.
 * ------------------------------------------------------------------------- */

/* Restart the decoder caches of the listed streams: stream h_streams[i]
 * starts again at position h_origin[i] exactly as rkv_state_init starts a
 * stream (same window and capacity, no valid rows); its ring rows stay in
 * memory but are no longer attended.  Other streams are untouched.
 * d_plan: NULL when the next call for these states is rkv_advance.  A
 * pipelined loop has already written the next step's plan: pass that plan,
 * and the listed streams are also advanced by that step and their entries of
 * d_plan rewritten, as if the restart had come before the launch that wrote
 * it.  The lists (host memory) are applied in order, so a stream listed twice
 * ends at its last origin; n = 0 does nothing.  Asynchronous on hip_stream
 * and allocation-free: the lists travel in kernel arguments (up to 64 streams
 * per launch) and the arrays may be reused as soon as the call returns.
 * Errors: RKV_EINVAL (null pointer with n > 0, n < 0, a stream index outside
 * [0, S)), RKV_ESTATE (an origin < 0), RKV_EALIGN (d_state not 8-byte or
 * d_plan not 16-byte aligned). */
int rkv_reset_streams(const rkv_cfg* cfg, rkv_stream_state* d_state, rkv_step_plan* d_plan,
                      int32_t n, const int32_t* h_streams, const int64_t* h_origin,
                      void* hip_stream);

#define RKV_STREAM_MAX_DECODE_KV 2000   /* the page's STREAM_MAX_DECODE_KV */

enum {
  RKV_RESTART_NONE = 0,
  RKV_RESTART_EOS = 1,
  RKV_RESTART_KV_OVERFLOW = 2,
  RKV_RESTART_NONTEXT_RUN = 3,
  RKV_RESTART_STALL = 4
};

/* Restart policy (host memory).  A step's token is text (id >=
 * text_token_min), a control token (0 <= id < text_token_min), or none
 * (id < 0).  Thresholds <= 0 (eos_token < 0) switch a condition off. */
typedef struct rkv_restart_cfg {
  int64_t max_decode_kv;   /* restart after the step that brings the decoder to
                              this many positions since its last restart, so no
                              step attends over more (RKV_STREAM_MAX_DECODE_KV) */
  int32_t eos_token;       /* restart after this token */
  int32_t text_token_min;  /* >= 0 */
  int32_t nontext_run;     /* restart after this many consecutive control tokens */
  int32_t stall_steps;     /* restart after this many consecutive steps without a token */
} rkv_restart_cfg;

/* Per-stream policy counters (host memory, all zero for a fresh stream). */
typedef struct rkv_restart_state {
  int64_t decode_len;  /* positions decoded since the last restart */
  int64_t restarts;    /* restarts so far */
  int32_t nontext;     /* current run of control tokens */
  int32_t idle;        /* current run of steps without a token */
} rkv_restart_state;

/* One clock step of the restart policy for num_streams streams: h_token[s]
 * is the token the decoder emitted for stream s at this step.  Updates
 * h_state[s]; writes h_reason[s] (RKV_RESTART_*; the first condition that
 * holds, in the page's order EOS, overflow, control-token run, stall) and the
 * indices of the streams to restart, increasing, to h_restart[0..count) (each
 * output may be NULL).  Returns count (>= 0), or RKV_EINVAL (null cfg, state
 * or token array, num_streams < 1, text_token_min < 0).  A restarted stream's
 * counters start over.  Host only: no device, no HIP call. */
int rkv_restart_step(const rkv_restart_cfg* cfg, rkv_restart_state* h_state,
                     int32_t num_streams, const int32_t* h_token, int32_t* h_reason,
                     int32_t* h_restart);

/* ---------------------------------------------------------------------------
 * Rolling log-mel front end (voxtral.c explainer, section 三: the mel buffer
 * rolls too -- audio samples that can no longer contribute to a future mel
 * frame are dropped -- so every stage runs in bounded memory).  The Audio8
 * explainer's file table gives the features: 16 kHz, 128 mel bands, hop 160
 * samples; one step of the 80 ms clock carries 1280 samples.
 * ------------------------------------------------------------------------- */

#define RKV_MEL_MAX_FFT 512

typedef struct rkv_mel_cfg {
  int32_t num_streams;       /* S >= 1 */
  int32_t n_fft;             /* analysis window in samples, hop <= n_fft <= RKV_MEL_MAX_FFT (400) */
  int32_t hop;               /* frame step in samples, >= 1 (160) */
  int32_t n_mels;            /* mel bands, 1 .. 1024 (128) */
  int32_t samples_per_step;  /* a multiple of hop and >= n_fft - hop (1280 at the 80 ms clock) */
  int32_t reserved;
} rkv_mel_cfg;

/* Slaney-scale triangular mel filterbank (linear below 1 kHz, logarithmic
 * above; filters spanning 0 Hz .. sample_rate / 2, each scaled by 2 / its
 * width in Hz) for bins k = 0 .. n_fft/2 at k * sample_rate / n_fft:
 * h_filters[n_mels][n_fft/2 + 1] (host, float32; float64 arithmetic).
 * RKV_EINVAL on a bad cfg, null pointer or sample_rate <= 0. */
int rkv_mel_filters_host(const rkv_mel_cfg* cfg, double sample_rate, float* h_filters);

/* One step of the rolling front end for every stream s.  The stream's buffer
 * is d_tail_in[s] (n_fft - hop samples kept from the previous step; zeros for
 * a new stream, which thus starts after n_fft - hop silent samples) followed
 * by d_samples[s] (samples_per_step new float32 samples).  For frames
 * f < samples_per_step / hop the frame is the buffer's samples
 * [f*hop, f*hop + n_fft) times the periodic Hann window
 * 0.5 - 0.5 cos(2 pi n / n_fft); out[s][f][m] =
 * log10(max(sum_k filters[m][k] |DFT_k(frame)|^2, 1e-10)) (float32; DFT sums
 * in float32).  d_tail_out[s] receives the n_fft - hop newest samples, all a
 * later frame can use.  Layouts: tails [S][n_fft - hop], samples
 * [S][samples_per_step], filters [n_mels][n_fft/2 + 1], out
 * [S][samples_per_step / hop][n_mels], all float32 device memory, 4-byte
 * aligned; d_tail_in and d_tail_out must not overlap (callers alternate two
 * buffers).  Asynchronous; no allocation.  RKV_EINVAL on a bad cfg, null
 * pointer or overlapping tails, RKV_EALIGN on misaligned pointers. */
int rkv_mel_step(const rkv_mel_cfg* cfg, const float* d_tail_in, float* d_tail_out,
                 const float* d_samples, const float* d_filters, float* d_out,
                 void* hip_stream);

/* ---------------------------------------------------------------------------
 * Incremental encoder step through a stack of layers (voxtral.c explainer,
 * section 三: the causal encoder computes only the new positions of a step,
 * each layer attending from them to its cached K/V).  Every layer is a
 * pre-norm residual block around the chunk attention:
 *   a = RMSNorm(x) g1;  x += Wo attn(a Wq^T, a Wk^T, a Wv^T);
 *   x += W2 gelu(W1 (RMSNorm(x) g2))
 * (RMSNorm(x) = x / sqrt(mean(x^2) + eps), exact erf GELU, no biases), with
 * the residual stream in float32 and the other activations in bfloat16.  The
 * layer structure beyond the attention is not given by the sources; the
 * synthetic weights make it a workload around the cache, not a model.
 * ------------------------------------------------------------------------- */

typedef struct rkv_encoder_cfg {
  int32_t ffn;        /* MLP width, a multiple of 64 (4 x hidden) */
  float norm_eps;     /* RMSNorm epsilon, >= 0 */
  int32_t reserved[2];
} rkv_encoder_cfg;

/* Bytes of one layer's bfloat16 weights; a stack is num_layers of them back to
 * back.  Per layer, in order: g1[hidden], wq, wk, wv, wo [hidden][hidden],
 * g2[hidden], w1[ffn][hidden], w2[hidden][ffn], each matrix with one row per
 * output feature; hidden = num_q_heads * head_dim.  0 on a bad cfg. */
size_t rkv_encoder_layer_weight_bytes(const rkv_cfg* cfg, const rkv_encoder_cfg* ec);

/* Workspace bytes of rkv_encoder_step for a cache of `slots` rows per head:
 * bfloat16 a, q, k, v, att [S*F][hidden] and u [S*F][ffn], float32 partial
 * sums [4][S*F][hidden] of the two products added into the residual stream
 * (computed in k-slices, added in slice order), plus the chunk attention's
 * workspace for one layer.  0 on a bad cfg. */
size_t rkv_encoder_step_workspace_bytes(const rkv_cfg* cfg, const rkv_encoder_cfg* ec,
                                        int32_t slots);

/* One clock step of cfg->num_layers encoder layers for every stream (ENC_CHUNK
 * mode, after rkv_advance: the plan is shared by all layers).  d_x [S][F][hidden]
 * float32 (device) holds the F new frames' embeddings on entry and the stack's
 * output on return.  Layer l reads weights at d_weights + l *
 * rkv_encoder_layer_weight_bytes() and appends to, and attends over, the
 * layer-l slice of the cache (kv->k + l * layer_stride, ...).  The launches
 * are asynchronous on hip_stream; no allocation.  Errors as for
 * rkv_encoder_chunk_attn, plus RKV_EINVAL for hidden or ffn not a multiple of
 * 64, hidden above 4096 or a mode other than ENC_CHUNK, RKV_EUNSUPPORTED for RKV_F_OUT_F32,
 * RKV_ESPACE for a short workspace and RKV_EALIGN for d_x, d_weights or
 * the workspace not 16-byte aligned. */
int rkv_encoder_step(const rkv_cfg* cfg, const rkv_encoder_cfg* ec, const rkv_step_plan* d_plan,
                     const rkv_kv_view* kv, const void* d_weights, float* d_x,
                     void* d_workspace, size_t workspace_bytes, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Delay conditioning (Audio8 ASR Infinite explainer, 可配置转写延迟; model
 * card, 优化操作点 and 架构).  The decoder is told how many clock steps it runs
 * behind real time, num_delay_tokens = target_delay_ms / clock; that count
 * as a sinusoidal embedding plus a learned frame-length embedding row is the
 * condition vector t_cond, which modulates the hidden state after the
 * attention of every decoder layer.  The sources do not give the form of the
 * modulation; it is taken here as a feature-wise scale and shift of the
 * layer's attention output (num_q_heads * head_dim features):
 *   h <- h (1 + gamma_l) + beta_l,   [gamma_l; beta_l] = A_l t_cond,
 *   t_cond = e(n) + table[frame_len],
 *   e_i = sin(n w_i), e_{D/2+i} = cos(n w_i), w_i = 10000^(-2i/D), i < D/2.
 * ------------------------------------------------------------------------- */

#define RKV_TCOND_MAX_CONDS 64
#define RKV_TCOND_MAX_DIM 1024

typedef struct rkv_tcond_cfg {
  int32_t num_layers;     /* L */
  int32_t hidden;         /* modulated features per row: a multiple of 8 */
  int32_t dim;            /* D: width of t_cond, even, 2 .. RKV_TCOND_MAX_DIM */
  int32_t num_conds;      /* C: distinct (delay, frame_len) settings, 1 .. RKV_TCOND_MAX_CONDS */
  int32_t max_frame_len;  /* the frame-length table has max_frame_len + 1 rows, >= 0 */
  int32_t reserved[3];
} rkv_tcond_cfg;

/* Host only: num_delay_tokens and frame_len (20 ms tower frames per step)
 * for a delay and an audio clock.  RKV_EINVAL for a clock other than 80, 120
 * or 160 ms, a delay that is not a positive integer multiple of the clock,
 * or a null output. */
int rkv_tcond_delay_tokens(int32_t target_delay_ms, int32_t clock_ms, int32_t* num_delay_tokens,
                           int32_t* frame_len);

/* Modulation vectors of every (layer, condition), once per change of the
 * settings (not per step): d_mod [L][C][2][hidden] float32 (device; gamma,
 * then beta) from h_num_delay[C] >= 0 and h_frame_len[C] in
 * [0, max_frame_len] (host arrays, passed in the launch), the frame-length
 * table d_frame_table [max_frame_len + 1][dim] and the matrices d_weights
 * [L][2 hidden][dim] (device, bfloat16; the gamma rows of A_l first).
 * t_cond in float32 from float64 sin/cos; products summed in float32.
 * Errors: RKV_EINVAL (bad cfg, null pointer, count or frame_len out of
 * range), RKV_EALIGN (a device pointer not 16-byte aligned), RKV_EHIP. */
int rkv_tcond_prepare(const rkv_tcond_cfg* tc, const int32_t* h_num_delay,
                      const int32_t* h_frame_len, const void* d_frame_table,
                      const void* d_weights, float* d_mod, void* hip_stream);

/* Per clock step, after the decoder attention: out <- out (1 + gamma) + beta,
 * in place, for every (layer, stream) row of d_out [L][S][num_q_heads]
 * [head_dim] (bfloat16, rounded to nearest even, or float32 with
 * RKV_F_OUT_F32), with the modulation of condition d_stream_cond[s] (device
 * int32 [S]).  A stream whose index lies outside [0, num_conds) is left as it
 * is (a negative index switches conditioning off for that stream).  tc must
 * match cfg: tc->num_layers == num_layers, tc->hidden == num_q_heads *
 * head_dim.  Errors: RKV_EINVAL (bad cfg or tc, mismatch, null pointer),
 * RKV_EALIGN (d_mod or d_out not 16-byte aligned), RKV_EHIP. */
int rkv_tcond_modulate(const rkv_cfg* cfg, const rkv_tcond_cfg* tc, const float* d_mod,
                       const int32_t* d_stream_cond, void* d_out, void* hip_stream);

/* The pipelined decode step with the delay conditioning applied as the
 * attention output is stored (Audio8 explainer, 可配置转写延迟: the condition
 * enters after each decoder layer's attention): bit-identical to
 * rkv_decode_step_pipelined followed by rkv_tcond_modulate with the same
 * d_mod and d_stream_cond, in one launch instead of two.  Arguments as
 * those two calls; REBASE and COMPACT modes (RKV_EINVAL for ENC_CHUNK), tc
 * matching cfg as for rkv_tcond_modulate. */
int rkv_decode_step_pipelined_tcond(const rkv_cfg* cfg, const rkv_tcond_cfg* tc,
                                    const float* d_mod, const int32_t* d_stream_cond,
                                    rkv_stream_state* d_state, const rkv_step_plan* d_plan,
                                    rkv_step_plan* d_plan_next, const rkv_kv_view* kv,
                                    const void* q, const void* k_new, const void* v_new,
                                    void* out, void* workspace, size_t workspace_bytes,
                                    void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* RKV_H */
