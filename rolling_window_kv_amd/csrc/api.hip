// C entry points of librkv: argument validation on the host, then kernel
// launches on the caller's stream.  Nothing here allocates device memory.

#include <math.h>
#include <string.h>

#include <mutex>

#include "rkv_internal.h"
#include "rkv_encoder.h"
#include "rkv_mel.h"
#include "rkv_tcond.h"
#include "rkv_update.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return RKV_OK;
  g_last_hip_error = (int)e;
  return RKV_EHIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_cfg(const rkv_cfg* c) {
  if (!c) return RKV_EINVAL;
  if (c->num_streams < 1 || c->num_layers < 1 || c->num_q_heads < 1 || c->num_kv_heads < 1)
    return RKV_EINVAL;
  if (c->head_dim != 64 && c->head_dim != 128) return RKV_EUNSUPPORTED;
  if (c->mode < RKV_MODE_REBASE || c->mode > RKV_MODE_ENC_CHUNK) return RKV_EUNSUPPORTED;
  if (c->flags &
      ~(uint32_t)(RKV_F_COMPENSATED | RKV_F_OUT_F32 | RKV_F_KV_FP16 | RKV_F_MERGE_LAUNCH))
    return RKV_EUNSUPPORTED;
  if (!(c->rope_base > 0.0) || !isfinite(c->rope_base)) return RKV_EINVAL;
  if (!(c->softmax_scale >= 0.0f) || !isfinite(c->softmax_scale)) return RKV_EINVAL;
  if (c->num_splits < 0) return RKV_EINVAL;
  if (c->num_q_heads % c->num_kv_heads) return RKV_EINVAL;
  const int64_t items = (int64_t)c->num_layers * c->num_streams * c->num_kv_heads;
  if (items * 64 > (int64_t)1 << 31) return RKV_EUNSUPPORTED;
  const int group = c->num_q_heads / c->num_kv_heads;
  switch (c->mode) {
    case RKV_MODE_REBASE:
      if (c->rebase_chunk < 1) return RKV_EINVAL;
      if (c->new_rows != 1) return RKV_EINVAL;
      if (group > RKV_MAX_GROUP) return RKV_EUNSUPPORTED;
      break;
    case RKV_MODE_COMPACT:
      if (c->new_rows != 1) return RKV_EINVAL;
      if (group > RKV_MAX_GROUP) return RKV_EUNSUPPORTED;
      if (c->flags & RKV_F_COMPENSATED) return RKV_EUNSUPPORTED;
      break;
    default:  // RKV_MODE_ENC_CHUNK
      if (c->num_q_heads != c->num_kv_heads) return RKV_EINVAL;
      if (c->new_rows < 1) return RKV_EINVAL;
      if (c->new_rows > RKV_MAX_NEW_ROWS) return RKV_EUNSUPPORTED;
      if (c->flags & (RKV_F_COMPENSATED | RKV_F_KV_FP16)) return RKV_EUNSUPPORTED;
      break;
  }
  return RKV_OK;
}

int check_kv(const rkv_cfg* c, const rkv_kv_view* kv) {
  if (!kv || !kv->k || !kv->v) return RKV_EINVAL;
  const bool comp = (c->flags & RKV_F_COMPENSATED) != 0;
  if (comp && !kv->k_lo) return RKV_EINVAL;
  if (kv->slots < 1 || c->max_cap < 1) return RKV_EINVAL;
  // every stream's capacity is at most max_cap (checked when the states were
  // built), so a ring of at least max_cap slots holds every row a plan names
  if (kv->slots < c->max_cap) return RKV_ESTATE;
  if (kv->slot_stride < c->head_dim || kv->layer_stride < 0 || kv->stream_stride < 0 ||
      kv->head_stride < 0)
    return RKV_EINVAL;
  if (!aligned16(kv->k) || !aligned16(kv->v) || (comp && !aligned16(kv->k_lo)))
    return RKV_EALIGN;
  if ((kv->layer_stride | kv->stream_stride | kv->head_stride | kv->slot_stride) & 7)
    return RKV_EALIGN;
  return RKV_OK;
}

int check_ptr(const void* p) {
  if (!p) return RKV_EINVAL;
  if (!aligned16(p)) return RKV_EALIGN;
  return RKV_OK;
}

rkv::RingArgs ring_of(const rkv_kv_view* kv) {
  rkv::RingArgs r;
  r.k = static_cast<uint16_t*>(kv->k);
  r.v = static_cast<uint16_t*>(kv->v);
  r.klo = static_cast<uint16_t*>(kv->k_lo);
  r.ls = kv->layer_stride;
  r.ss = kv->stream_stride;
  r.hs = kv->head_stride;
  r.rs = kv->slot_stride;
  r.slots = kv->slots;
  return r;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Workspace of a split launch: one merge counter per item (zero between
// calls), then the float32 partials [item][split][16 + 8 d].
size_t ticket_bytes(const rkv_cfg* c) {
  return align256((size_t)c->num_layers * c->num_streams * c->num_kv_heads * sizeof(uint32_t));
}
size_t partial_bytes(const rkv_cfg* c, int32_t slots) {
  const int n = rkv::choose_splits(c, slots);
  if (n <= 1) return 0;
  const int64_t items = (int64_t)c->num_layers * c->num_streams * c->num_kv_heads;
  return (size_t)(items * n * rkv::partial_floats(c->head_dim) * (int64_t)sizeof(float));
}
size_t workspace_for(const rkv_cfg* c, int32_t slots) {
  const size_t p = partial_bytes(c, slots);
  return p ? ticket_bytes(c) + p : 0;
}

// Device array for the allocation-free entry point: each GPU the library
// runs on holds its own copy until the process ends.  Host code never uses
// the array's name as an address (in host code it is only a stand-in): the
// device address comes from hipGetSymbolAddress, looked up once per device.
// Its last kScratchTicketBytes hold the merge counters (one per item, zero
// at load and after every call), the rest the split partials, so counters
// never land where an earlier call with another configuration left partials.
constexpr size_t kScratchBytes = RKV_NOALLOC_SCRATCH_BYTES;
constexpr size_t kScratchTicketBytes = (size_t)RKV_NOALLOC_MAX_SPLIT_ITEMS * sizeof(uint32_t);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The scratch array's device address on the current device.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return RKV_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!p) return RKV_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RKV_OK;
}

// Workgroups that pull an encoder step's next weights into the cache during
// a chunk-attention launch (one per CU).
constexpr int kPullBlocks = 256;

// ws == kUseScratch: the split partials go to the library's scratch array
// (after every argument check, so errors still come before any HIP call).
void* const kUseScratch = reinterpret_cast<void*>(~(uintptr_t)0);

int attention(const rkv_cfg* cfg, rkv::AttnKind kind, const rkv_step_plan* plan,
              const rkv_kv_view* kv, const void* q, const void* knew, const void* vnew,
              void* out, void* ws, size_t ws_bytes, void* stream,
              rkv_stream_state* next_state = nullptr, rkv_step_plan* next_plan = nullptr,
              const void* pull = nullptr, size_t pull_bytes = 0,
              const float* tc_mod = nullptr, const int32_t* tc_cond = nullptr,
              int32_t tc_conds = 0) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (next_state || next_plan) {
    if (!next_state || !next_plan || !plan) return RKV_EINVAL;
    if (((uintptr_t)next_state & 7u) || !aligned16(next_plan)) return RKV_EALIGN;
    // the plan being read and the plan being written must not overlap
    const uintptr_t a0 = (uintptr_t)plan, b0 = (uintptr_t)next_plan;
    const uintptr_t n = sizeof(rkv_step_plan) * (uintptr_t)cfg->num_streams;
    if (a0 < b0 + n && b0 < a0 + n) return RKV_EINVAL;
  }
  if (kind == rkv::kEncoderFused && cfg->mode != RKV_MODE_ENC_CHUNK) return RKV_EINVAL;
  if (kind != rkv::kEncoderFused && cfg->mode == RKV_MODE_ENC_CHUNK) return RKV_EINVAL;
  if ((rc = check_kv(cfg, kv))) return rc;
  if (!plan) return RKV_EINVAL;
  if ((rc = check_ptr(q)) || (rc = check_ptr(out))) return rc;
  if (kind != rkv::kDecodeRead && ((rc = check_ptr(knew)) || (rc = check_ptr(vnew)))) return rc;
  const size_t need = workspace_for(cfg, kv->slots);
  float* partials = nullptr;
  uint32_t* tickets = nullptr;
  if (ws == kUseScratch) {
    const size_t pbytes = partial_bytes(cfg, kv->slots);
    const int64_t items = (int64_t)cfg->num_layers * cfg->num_streams * cfg->num_kv_heads;
    if (pbytes &&
        (pbytes > kScratchBytes - kScratchTicketBytes || items > RKV_NOALLOC_MAX_SPLIT_ITEMS))
      return RKV_ESPACE;
    void* base = nullptr;
    if (pbytes && (rc = scratch_address(&base))) return rc;
    if (pbytes) {
      partials = static_cast<float*>(base);
      tickets = reinterpret_cast<uint32_t*>(static_cast<char*>(base) + kScratchBytes -
                                            kScratchTicketBytes);
    }
  } else if (need) {
    if (!ws || ws_bytes < need) return RKV_ESPACE;
    if (!aligned16(ws)) return RKV_EALIGN;
    tickets = static_cast<uint32_t*>(ws);
    partials = reinterpret_cast<float*>(static_cast<char*>(ws) + ticket_bytes(cfg));
  }
  rkv::AttnArgs a;
  a.plan = plan;
  a.ring = ring_of(kv);
  a.q = static_cast<const uint16_t*>(q);
  a.knew = static_cast<const uint16_t*>(knew);
  a.vnew = static_cast<const uint16_t*>(vnew);
  a.out = out;
  a.ws = partials;
  a.nsplit = rkv::choose_splits(cfg, kv->slots);
  // The splits merge inside the attention launch when its workgroups fit in
  // one round on the chip (latency-bound launches: one layer, few streams);
  // a launch of several rounds merges in a second launch, because there the
  // waves that wait for the hand-over hold slots other workgroups would
  // stream in (26 x 16 compaction, 3 splits: 589 against 562 us a step).
  const int64_t blocks = (int64_t)cfg->num_layers * cfg->num_streams * cfg->num_kv_heads *
                         a.nsplit;
  a.tickets = ((cfg->flags & RKV_F_MERGE_LAUNCH) || blocks > rkv::kMergeInLaunchMaxBlocks)
                  ? nullptr
                  : tickets;
  a.S = cfg->num_streams;
  a.L = cfg->num_layers;
  a.Hkv = cfg->num_kv_heads;
  a.G = kind == rkv::kEncoderFused ? cfg->new_rows : cfg->num_q_heads / cfg->num_kv_heads;
  a.F = cfg->new_rows;
  a.out_f32 = (cfg->flags & RKV_F_OUT_F32) ? 1 : 0;
  const double scale =
      cfg->softmax_scale > 0.0f ? (double)cfg->softmax_scale : 1.0 / sqrt((double)cfg->head_dim);
  a.scale_log2 = (float)(scale * 1.4426950408889634);
  a.adv_state = next_state;
  a.adv_plan = next_plan;
  a.adv_mode = cfg->mode;
  a.adv_dc = cfg->rebase_chunk;
  a.adv_F = cfg->new_rows;
  a.adv_half = cfg->head_dim / 2;
  a.adv_theta = rkv::theta_table(cfg);
  const bool pulls = kind == rkv::kEncoderFused && pull && pull_bytes >= 16;
  a.pull = pulls ? static_cast<const char*>(pull) : nullptr;
  a.pull_bytes = pulls ? (int64_t)(pull_bytes & ~(size_t)15) : 0;
  a.pull_blocks = pulls ? kPullBlocks : 0;
  const bool tcond = kind != rkv::kEncoderFused && tc_mod && tc_cond && tc_conds > 0;
  a.tc_mod = tcond ? tc_mod : nullptr;
  a.tc_cond = tcond ? tc_cond : nullptr;
  a.tc_conds = tcond ? tc_conds : 0;
  return hip_status(rkv::launch_attention(cfg, kind, a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int rkv_version(void) { return RKV_VERSION; }

const char* rkv_strerror(int status) {
  switch (status) {
    case RKV_OK: return "ok";
    case RKV_EINVAL: return "invalid argument";
    case RKV_EUNSUPPORTED: return "unsupported configuration";
    case RKV_EALIGN: return "pointer or stride not 16-byte aligned";
    case RKV_ESTATE: return "stream state inconsistent with the mode";
    case RKV_EHIP: return "HIP launch failed";
    case RKV_ESPACE: return "workspace too small";
    default: return "unknown status";
  }
}

int rkv_last_hip_error(void) { return g_last_hip_error; }

int rkv_validate_cfg(const rkv_cfg* cfg) { return check_cfg(cfg); }

int rkv_state_init_host(const rkv_cfg* cfg, const int32_t* h_window, const int32_t* h_cap,
                        const int64_t* h_origin, rkv_stream_state* h_state) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!h_window || !h_cap || !h_origin || !h_state) return RKV_EINVAL;
  if (cfg->max_cap < 1) return RKV_EINVAL;
  for (int s = 0; s < cfg->num_streams; ++s) {
    const int32_t W = h_window[s], cap = h_cap[s];
    const int64_t origin = h_origin[s];
    if (W < 1 || cap < 1 || origin < 0 || cap > cfg->max_cap) return RKV_ESTATE;
    switch (cfg->mode) {
      case RKV_MODE_REBASE:
        if (cap != W) return RKV_ESTATE;
        break;
      case RKV_MODE_COMPACT:
        if (cap <= W) return RKV_ESTATE;
        break;
      default:
        if (cap < W + cfg->new_rows) return RKV_ESTATE;
        break;
    }
  }
  for (int s = 0; s < cfg->num_streams; ++s)
    h_state[s] = rkv::initial_state(h_origin[s], h_window[s], h_cap[s], cfg->mode,
                                    cfg->rebase_chunk);
  return RKV_OK;
}

int rkv_state_advance_host(const rkv_cfg* cfg, rkv_stream_state* h_state, int64_t steps) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!h_state || steps < 0) return RKV_EINVAL;
  if (cfg->max_cap < 1) return RKV_EINVAL;
  for (int s = 0; s < cfg->num_streams; ++s) {
    const rkv_stream_state& x = h_state[s];
    if (x.window < 1 || x.cap < 1 || x.cap > cfg->max_cap || x.len < 0 || x.len > x.cap ||
        x.origin < 0 || x.t < x.origin - 1)
      return RKV_ESTATE;
    switch (cfg->mode) {
      case RKV_MODE_REBASE:
        if (x.cap != x.window) return RKV_ESTATE;
        break;
      case RKV_MODE_COMPACT:
        if (x.cap <= x.window) return RKV_ESTATE;
        break;
      default:
        if (x.cap < x.window + cfg->new_rows) return RKV_ESTATE;
        break;
    }
  }
  for (int s = 0; s < cfg->num_streams; ++s)
    for (int64_t i = 0; i < steps; ++i)
      h_state[s] = rkv::make_plan(h_state[s], cfg->mode, cfg->rebase_chunk, cfg->new_rows).next;
  return RKV_OK;
}

int rkv_state_init(const rkv_cfg* cfg, rkv_stream_state* d_state, const int32_t* h_window,
                   const int32_t* h_cap, const int64_t* h_origin, void* hip_stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!d_state || !h_window || !h_cap || !h_origin) return RKV_EINVAL;
  if ((uintptr_t)d_state & 7u) return RKV_EALIGN;
  // Built in host chunks on the stack and copied in stream order; the call
  // returns once the copies are done, so the caller's arrays may be reused.
  constexpr int kChunk = 128;
  rkv_stream_state buf[kChunk];
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  rkv_cfg sub = *cfg;
  for (int s0 = 0; s0 < cfg->num_streams; s0 += kChunk) {
    sub.num_streams = cfg->num_streams - s0 < kChunk ? cfg->num_streams - s0 : kChunk;
    rc = rkv_state_init_host(&sub, h_window + s0, h_cap + s0, h_origin + s0, buf);
    if (rc) return rc;
    hipError_t e = hipMemcpyAsync(d_state + s0, buf, sizeof(rkv_stream_state) * sub.num_streams,
                                  hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_status(e);
  }
  return RKV_OK;
}

int rkv_reset_streams(const rkv_cfg* cfg, rkv_stream_state* d_state, rkv_step_plan* d_plan,
                      int32_t n, const int32_t* h_streams, const int64_t* h_origin,
                      void* hip_stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!d_state || n < 0) return RKV_EINVAL;
  if (n > 0 && (!h_streams || !h_origin)) return RKV_EINVAL;
  if ((uintptr_t)d_state & 7u) return RKV_EALIGN;
  if (d_plan && !aligned16(d_plan)) return RKV_EALIGN;
  for (int32_t i = 0; i < n; ++i) {
    if (h_streams[i] < 0 || h_streams[i] >= cfg->num_streams) return RKV_EINVAL;
    if (h_origin[i] < 0) return RKV_ESTATE;
  }
  // Launches of at most ResetList::kMax streams, in list order; a launch ends
  // before a stream already in it, so each launch resets distinct streams and
  // a repeated stream takes its later origin.
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  rkv::ResetList list;
  list.n = 0;
  for (int32_t i = 0; i <= n; ++i) {
    bool flush = i == n || list.n == rkv::ResetList::kMax;
    for (int j = 0; !flush && j < list.n; ++j) flush = list.stream[j] == h_streams[i];
    if (flush && list.n > 0) {
      hipError_t e = rkv::launch_reset(cfg, d_state, d_plan, list, stream);
      if (e != hipSuccess) return hip_status(e);
      list.n = 0;
    }
    if (i < n) {
      list.stream[list.n] = h_streams[i];
      list.origin[list.n] = h_origin[i];
      ++list.n;
    }
  }
  return RKV_OK;
}

static int check_mel(const rkv_mel_cfg* c) {
  if (!c) return RKV_EINVAL;
  if (c->num_streams < 1 || c->hop < 1 || c->n_fft < c->hop || c->n_fft > RKV_MEL_MAX_FFT)
    return RKV_EINVAL;
  if (c->n_mels < 1 || c->n_mels > 1024) return RKV_EINVAL;
  if (c->samples_per_step < 1 || c->samples_per_step % c->hop ||
      c->samples_per_step < c->n_fft - c->hop)
    return RKV_EINVAL;
  const int64_t frames = (int64_t)c->num_streams * (c->samples_per_step / c->hop);
  if (c->samples_per_step / c->hop > 65535 || frames > ((int64_t)1 << 31)) return RKV_EINVAL;
  return RKV_OK;
}

int rkv_mel_filters_host(const rkv_mel_cfg* cfg, double sample_rate, float* h_filters) {
  int rc = check_mel(cfg);
  if (rc) return rc;
  if (!h_filters || !(sample_rate > 0.0) || !isfinite(sample_rate)) return RKV_EINVAL;
  // Slaney mel scale: 200/3 Hz per mel up to 1 kHz (15 mel), then a fixed
  // ratio of 6.4 per 27 mel.
  const double f_sp = 200.0 / 3.0, min_log_hz = 1000.0, min_log_mel = min_log_hz / f_sp;
  const double step = log(6.4) / 27.0;
  auto to_mel = [&](double f) {
    return f < min_log_hz ? f / f_sp : min_log_mel + log(f / min_log_hz) / step;
  };
  auto to_hz = [&](double m) {
    return m < min_log_mel ? m * f_sp : min_log_hz * exp(step * (m - min_log_mel));
  };
  const int bins = cfg->n_fft / 2 + 1;
  const double top = to_mel(sample_rate / 2.0);
  for (int b = 0; b < cfg->n_mels; ++b) {
    const double lo = to_hz(top * b / (cfg->n_mels + 1));
    const double mid = to_hz(top * (b + 1) / (cfg->n_mels + 1));
    const double hi = to_hz(top * (b + 2) / (cfg->n_mels + 1));
    const double scale = 2.0 / (hi - lo);
    for (int k = 0; k < bins; ++k) {
      const double f = k * sample_rate / cfg->n_fft;
      const double up = (f - lo) / (mid - lo), down = (hi - f) / (hi - mid);
      const double t = up < down ? up : down;
      h_filters[(int64_t)b * bins + k] = (float)((t > 0.0 ? t : 0.0) * scale);
    }
  }
  return RKV_OK;
}

int rkv_mel_step(const rkv_mel_cfg* cfg, const float* d_tail_in, float* d_tail_out,
                 const float* d_samples, const float* d_filters, float* d_out,
                 void* hip_stream) {
  int rc = check_mel(cfg);
  if (rc) return rc;
  if (!d_tail_in || !d_tail_out || !d_samples || !d_filters || !d_out) return RKV_EINVAL;
  const uintptr_t a = (uintptr_t)d_tail_in, b = (uintptr_t)d_tail_out;
  const uintptr_t bytes = (uintptr_t)cfg->num_streams * (cfg->n_fft - cfg->hop) * sizeof(float);
  if (bytes && a < b + bytes && b < a + bytes) return RKV_EINVAL;
  if ((a | b | (uintptr_t)d_samples | (uintptr_t)d_filters | (uintptr_t)d_out) & 3u)
    return RKV_EALIGN;
  return hip_status(rkv::launch_mel(cfg, d_tail_in, d_tail_out, d_samples, d_filters, d_out,
                                    static_cast<hipStream_t>(hip_stream)));
}

size_t rkv_workspace_bytes(const rkv_cfg* cfg, int32_t slots) {
  if (check_cfg(cfg) || slots < 1) return 0;
  return workspace_for(cfg, slots);
}

int rkv_advance(const rkv_cfg* cfg, rkv_stream_state* d_state, rkv_step_plan* d_plan,
                void* hip_stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!d_state || !d_plan) return RKV_EINVAL;
  if (((uintptr_t)d_state & 7u) || !aligned16(d_plan)) return RKV_EALIGN;
  return hip_status(rkv::launch_advance(cfg, d_state, d_plan, static_cast<hipStream_t>(hip_stream)));
}

int rkv_append(const rkv_cfg* cfg, const rkv_step_plan* d_plan, const rkv_kv_view* kv,
               const void* k_new, const void* v_new, void* hip_stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if ((rc = check_kv(cfg, kv))) return rc;
  if (!d_plan) return RKV_EINVAL;
  if ((rc = check_ptr(k_new)) || (rc = check_ptr(v_new))) return rc;
  return hip_status(rkv::launch_append(cfg, d_plan, ring_of(kv), static_cast<const uint16_t*>(k_new),
                                       static_cast<const uint16_t*>(v_new),
                                       static_cast<hipStream_t>(hip_stream)));
}

int rkv_roll_rebase(const rkv_cfg* cfg, const rkv_step_plan* d_plan, const rkv_kv_view* kv,
                    void* hip_stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (cfg->mode != RKV_MODE_REBASE) return RKV_EINVAL;
  if ((rc = check_kv(cfg, kv))) return rc;
  if (!d_plan) return RKV_EINVAL;
  return hip_status(rkv::launch_rebase(cfg, d_plan, ring_of(kv), static_cast<hipStream_t>(hip_stream)));
}

int rkv_update_step(const rkv_cfg* cfg, const rkv_step_plan* d_plan, const rkv_kv_view* kv,
                    const void* k_new, const void* v_new, void* hip_stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if ((rc = check_kv(cfg, kv))) return rc;
  if (!d_plan) return RKV_EINVAL;
  if ((rc = check_ptr(k_new)) || (rc = check_ptr(v_new))) return rc;
  return hip_status(rkv::launch_update(cfg, d_plan, ring_of(kv), static_cast<const uint16_t*>(k_new),
                                       static_cast<const uint16_t*>(v_new),
                                       static_cast<hipStream_t>(hip_stream)));
}

int rkv_compact(const rkv_cfg* cfg, const rkv_step_plan* d_plan, const rkv_kv_view* kv,
                void* hip_stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (cfg->mode != RKV_MODE_COMPACT) return RKV_EINVAL;
  if ((rc = check_kv(cfg, kv))) return rc;
  if (!d_plan) return RKV_EINVAL;
  return hip_status(rkv::launch_compact(cfg, d_plan, ring_of(kv), static_cast<hipStream_t>(hip_stream)));
}

int rkv_decode_attn(const rkv_cfg* cfg, const rkv_step_plan* d_plan, const rkv_kv_view* kv,
                    const void* q, void* out, void* workspace, size_t workspace_bytes,
                    void* hip_stream) {
  return attention(cfg, rkv::kDecodeRead, d_plan, kv, q, nullptr, nullptr, out, workspace,
                   workspace_bytes, hip_stream);
}

int rkv_decode_step(const rkv_cfg* cfg, const rkv_step_plan* d_plan, const rkv_kv_view* kv,
                    const void* q, const void* k_new, const void* v_new, void* out,
                    void* workspace, size_t workspace_bytes, void* hip_stream) {
  return attention(cfg, rkv::kDecodeFused, d_plan, kv, q, k_new, v_new, out, workspace,
                   workspace_bytes, hip_stream);
}

int rkv_decode_step_noalloc(const rkv_cfg* cfg, const rkv_step_plan* d_plan,
                            const rkv_kv_view* kv, const void* q, const void* k_new,
                            const void* v_new, void* out, void* hip_stream) {
  return attention(cfg, rkv::kDecodeFused, d_plan, kv, q, k_new, v_new, out, kUseScratch, 0,
                   hip_stream);
}

int rkv_decode_step_pipelined(const rkv_cfg* cfg, rkv_stream_state* d_state,
                              const rkv_step_plan* d_plan, rkv_step_plan* d_plan_next,
                              const rkv_kv_view* kv, const void* q, const void* k_new,
                              const void* v_new, void* out, void* workspace,
                              size_t workspace_bytes, void* hip_stream) {
  return attention(cfg, rkv::kDecodeFused, d_plan, kv, q, k_new, v_new, out, workspace,
                   workspace_bytes, hip_stream, d_state, d_plan_next);
}

int rkv_decode_attn_pipelined(const rkv_cfg* cfg, rkv_stream_state* d_state,
                              const rkv_step_plan* d_plan, rkv_step_plan* d_plan_next,
                              const rkv_kv_view* kv, const void* q, void* out, void* workspace,
                              size_t workspace_bytes, void* hip_stream) {
  if (cfg && cfg->mode == RKV_MODE_ENC_CHUNK) return RKV_EINVAL;
  return attention(cfg, rkv::kDecodeRead, d_plan, kv, q, nullptr, nullptr, out, workspace,
                   workspace_bytes, hip_stream, d_state, d_plan_next);
}

static int check_encoder(const rkv_cfg* cfg, const rkv_encoder_cfg* ec) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!ec || cfg->mode != RKV_MODE_ENC_CHUNK) return RKV_EINVAL;
  // the attention output is a bfloat16 activation of the stack
  if (cfg->flags & RKV_F_OUT_F32) return RKV_EUNSUPPORTED;
  const int hidden = cfg->num_q_heads * cfg->head_dim;
  if (hidden % 64 || hidden > rkv::kEncoderMaxHidden || ec->ffn < 64 || ec->ffn % 64)
    return RKV_EINVAL;
  if (!(ec->norm_eps >= 0.0f) || !isfinite(ec->norm_eps)) return RKV_EINVAL;
  return RKV_OK;
}

static size_t encoder_layer_elems(const rkv_cfg* cfg, const rkv_encoder_cfg* ec) {
  const size_t h = (size_t)cfg->num_q_heads * cfg->head_dim, f = (size_t)ec->ffn;
  return 2 * h + 4 * h * h + 2 * h * f;
}


size_t rkv_encoder_layer_weight_bytes(const rkv_cfg* cfg, const rkv_encoder_cfg* ec) {
  if (check_encoder(cfg, ec)) return 0;
  return 2 * encoder_layer_elems(cfg, ec);
}

// k-slices of the two products that add into the residual stream (the
// output projection and the MLP's second product): their float32 partial
// sums are added, in slice order, by the RMSNorm launch that reads x next.
static int encoder_splits(int K) {
  const int stages = K / 64;
  return stages % 4 == 0 ? 4 : stages % 2 == 0 ? 2 : 1;
}

size_t rkv_encoder_step_workspace_bytes(const rkv_cfg* cfg, const rkv_encoder_cfg* ec,
                                        int32_t slots) {
  if (check_encoder(cfg, ec) || slots < 1) return 0;
  const size_t tokens = (size_t)cfg->num_streams * cfg->new_rows;
  const size_t h = (size_t)cfg->num_q_heads * cfg->head_dim;
  rkv_cfg one = *cfg;
  one.num_layers = 1;
  return 5 * align256(2 * tokens * h) + align256(2 * tokens * ec->ffn) +
         align256(4 * rkv::kGemmMaxSet * tokens * h) + align256(workspace_for(&one, slots));
}

int rkv_encoder_step(const rkv_cfg* cfg, const rkv_encoder_cfg* ec, const rkv_step_plan* d_plan,
                     const rkv_kv_view* kv, const void* d_weights, float* d_x,
                     void* d_workspace, size_t workspace_bytes, void* hip_stream) {
  int rc = check_encoder(cfg, ec);
  if (rc) return rc;
  if ((rc = check_kv(cfg, kv))) return rc;
  if (!d_plan || !d_weights || !d_x || !d_workspace) return RKV_EINVAL;
  if (!aligned16(d_weights) || !aligned16(d_x) || !aligned16(d_workspace)) return RKV_EALIGN;
  const size_t need = rkv_encoder_step_workspace_bytes(cfg, ec, kv->slots);
  if (workspace_bytes < need) return RKV_ESPACE;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const int M = cfg->num_streams * cfg->new_rows;
  const int H = cfg->num_q_heads * cfg->head_dim, FF = ec->ffn;
  const float eps = ec->norm_eps;
  // workspace: bfloat16 a, q, k, v, att [M][H], u [M][FF]; float32 partial
  // sums [kGemmMaxSet][M][H]; then the chunk attention's own workspace
  char* p = static_cast<char*>(d_workspace);
  const size_t act = align256((size_t)2 * M * H);
  uint16_t* a = reinterpret_cast<uint16_t*>(p);
  uint16_t* q = reinterpret_cast<uint16_t*>(p + act);
  uint16_t* k = reinterpret_cast<uint16_t*>(p + 2 * act);
  uint16_t* v = reinterpret_cast<uint16_t*>(p + 3 * act);
  uint16_t* att = reinterpret_cast<uint16_t*>(p + 4 * act);
  uint16_t* u = reinterpret_cast<uint16_t*>(p + 5 * act);
  float* part = reinterpret_cast<float*>(p + 5 * act + align256((size_t)2 * M * FF));
  const size_t head = 5 * act + align256((size_t)2 * M * FF) +
                      align256((size_t)4 * rkv::kGemmMaxSet * M * H);
  void* aws = p + head;
  const size_t aws_bytes = workspace_bytes - head;
  const int64_t part_stride = (int64_t)M * H;
  rkv_cfg one = *cfg;
  one.num_layers = 1;
  // split partials (few streams) merged by a second launch: the merge
  // counters of an in-launch merge would need a zeroed workspace
  one.flags |= RKV_F_MERGE_LAUNCH;
  const size_t layer_elems = encoder_layer_elems(cfg, ec);
  const int so = encoder_splits(H), s2 = encoder_splits(FF);
  hipError_t e;
  int pending = 0;            // partial sums of the previous product not yet in x
  for (int l = 0; l < cfg->num_layers; ++l) {
    const uint16_t* w = static_cast<const uint16_t*>(d_weights) + (size_t)l * layer_elems;
    const uint16_t* g1 = w;
    const uint16_t* wq = g1 + H;
    const uint16_t* wk = wq + (size_t)H * H;
    const uint16_t* wv = wk + (size_t)H * H;
    const uint16_t* wo = wv + (size_t)H * H;
    const uint16_t* g2 = wo + (size_t)H * H;
    const uint16_t* w1 = g2 + H;
    const uint16_t* w2 = w1 + (size_t)FF * H;
    // x += previous layer's MLP output; a = RMSNorm(x) g1
    if ((e = rkv::launch_rmsnorm(d_x, part, pending, part_stride, g1, a, M, H, eps, stream)) !=
        hipSuccess)
      return hip_status(e);
    const uint16_t* wqkv[3] = {wq, wk, wv};
    const uint16_t* aaa[3] = {a, a, a};
    void* cqkv[3] = {q, k, v};
    if ((e = rkv::launch_gemm(rkv::GemmEpilogue::kStoreBf16, wqkv, aaa, cqkv, 3, M, H, H, H,
                              stream)) != hipSuccess)
      return hip_status(e);
    rkv_kv_view lv = *kv;
    lv.k = static_cast<uint16_t*>(kv->k) + (size_t)l * kv->layer_stride;
    lv.v = static_cast<uint16_t*>(kv->v) + (size_t)l * kv->layer_stride;
    // While the attention streams this layer's window, its extra workgroups
    // pull the weights of the next four products into the infinity cache:
    // Wo, g2, W1, W2 of this layer and g1, Wq, Wk, Wv of the next, which lie
    // back to back (a product reading its weights cold from HBM is limited by
    // the first touch of each weight panel: q/k/v 14.1 against 11.6 us).
    const size_t pull_elems = (size_t)H * H + H + 2 * (size_t)FF * H +
                              (l + 1 < cfg->num_layers ? H + 3 * (size_t)H * H : 0);
    if ((rc = attention(&one, rkv::kEncoderFused, d_plan, &lv, q, k, v, att, aws, aws_bytes,
                        hip_stream, nullptr, nullptr, wo, 2 * pull_elems)))
      return rc;
    // output projection in `so` k-slices; x += their sum, a = RMSNorm(x) g2
    const uint16_t* ws_[rkv::kGemmMaxSet];
    const uint16_t* xs_[rkv::kGemmMaxSet];
    void* cs_[rkv::kGemmMaxSet];
    for (int i = 0; i < so; ++i) {
      ws_[i] = wo + (size_t)i * (H / so);
      xs_[i] = att + (size_t)i * (H / so);
      cs_[i] = part + i * part_stride;
    }
    if ((e = rkv::launch_gemm(rkv::GemmEpilogue::kStoreF32, ws_, xs_, cs_, so, M, H, H / so, H,
                              stream)) != hipSuccess)
      return hip_status(e);
    if ((e = rkv::launch_rmsnorm(d_x, part, so, part_stride, g2, a, M, H, eps, stream)) !=
        hipSuccess)
      return hip_status(e);
    const uint16_t* w1s[1] = {w1};
    const uint16_t* as[1] = {a};
    void* us[1] = {u};
    if ((e = rkv::launch_gemm(rkv::GemmEpilogue::kGeluBf16, w1s, as, us, 1, M, FF, H, H,
                              stream)) != hipSuccess)
      return hip_status(e);
    for (int i = 0; i < s2; ++i) {
      ws_[i] = w2 + (size_t)i * (FF / s2);
      xs_[i] = u + (size_t)i * (FF / s2);
      cs_[i] = part + i * part_stride;
    }
    if ((e = rkv::launch_gemm(rkv::GemmEpilogue::kStoreF32, ws_, xs_, cs_, s2, M, H, FF / s2, FF,
                              stream)) != hipSuccess)
      return hip_status(e);
    pending = s2;
  }
  // the last layer's MLP output into x
  if ((e = rkv::launch_rmsnorm(d_x, part, pending, part_stride, nullptr, nullptr, M, H, eps,
                               stream)) != hipSuccess)
    return hip_status(e);
  return RKV_OK;
}

int rkv_encoder_chunk_attn(const rkv_cfg* cfg, const rkv_step_plan* d_plan,
                           const rkv_kv_view* kv, const void* q, const void* k_new,
                           const void* v_new, void* out, void* workspace,
                           size_t workspace_bytes, void* hip_stream) {
  return attention(cfg, rkv::kEncoderFused, d_plan, kv, q, k_new, v_new, out, workspace,
                   workspace_bytes, hip_stream);
}

}  // extern "C"

static_assert(sizeof(rkv_cfg) == 56, "rkv_cfg layout");
static_assert(sizeof(rkv_stream_state) == 48, "rkv_stream_state layout");
static_assert(offsetof(rkv_step_plan, rope_new) == 128, "rkv_step_plan header");
static_assert(sizeof(rkv_step_plan) == 128 + 8192 + 1024, "rkv_step_plan layout");
static_assert(sizeof(rkv_kv_view) == 64, "rkv_kv_view layout");

// ---------------------------------------------------------------------------
// Delay conditioning
// ---------------------------------------------------------------------------

static int check_tcond(const rkv_tcond_cfg* tc) {
  if (!tc) return RKV_EINVAL;
  if (tc->num_layers < 1 || tc->hidden < 8 || tc->hidden % 8) return RKV_EINVAL;
  if (tc->dim < 2 || tc->dim % 2 || tc->dim > RKV_TCOND_MAX_DIM) return RKV_EINVAL;
  if (tc->num_conds < 1 || tc->num_conds > RKV_TCOND_MAX_CONDS) return RKV_EINVAL;
  if (tc->max_frame_len < 0 || tc->max_frame_len > (1 << 16)) return RKV_EINVAL;
  return RKV_OK;
}

int rkv_tcond_delay_tokens(int32_t target_delay_ms, int32_t clock_ms, int32_t* num_delay_tokens,
                           int32_t* frame_len) {
  if (!num_delay_tokens || !frame_len) return RKV_EINVAL;
  if (clock_ms != 80 && clock_ms != 120 && clock_ms != 160) return RKV_EINVAL;
  if (target_delay_ms <= 0 || target_delay_ms % clock_ms) return RKV_EINVAL;
  *num_delay_tokens = target_delay_ms / clock_ms;
  *frame_len = clock_ms / 20;
  return RKV_OK;
}

int rkv_tcond_prepare(const rkv_tcond_cfg* tc, const int32_t* h_num_delay,
                      const int32_t* h_frame_len, const void* d_frame_table,
                      const void* d_weights, float* d_mod, void* hip_stream) {
  int rc = check_tcond(tc);
  if (rc) return rc;
  if (!h_num_delay || !h_frame_len) return RKV_EINVAL;
  if ((rc = check_ptr(d_frame_table)) || (rc = check_ptr(d_weights)) || (rc = check_ptr(d_mod)))
    return rc;
  rkv::TcondConds conds{};
  for (int c = 0; c < tc->num_conds; ++c) {
    if (h_num_delay[c] < 0 || h_num_delay[c] > (1 << 24)) return RKV_EINVAL;
    if (h_frame_len[c] < 0 || h_frame_len[c] > tc->max_frame_len) return RKV_EINVAL;
    conds.num_delay[c] = h_num_delay[c];
    conds.frame_len[c] = h_frame_len[c];
  }
  return hip_status(rkv::launch_tcond_prepare(tc, conds, static_cast<const uint16_t*>(d_frame_table),
                                              static_cast<const uint16_t*>(d_weights), d_mod,
                                              static_cast<hipStream_t>(hip_stream)));
}

int rkv_tcond_modulate(const rkv_cfg* cfg, const rkv_tcond_cfg* tc, const float* d_mod,
                       const int32_t* d_stream_cond, void* d_out, void* hip_stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if ((rc = check_tcond(tc))) return rc;
  const int hidden = cfg->num_q_heads * cfg->head_dim;
  if (tc->num_layers != cfg->num_layers || tc->hidden != hidden) return RKV_EINVAL;
  if (!d_stream_cond) return RKV_EINVAL;
  if ((rc = check_ptr(d_mod)) || (rc = check_ptr(d_out))) return rc;
  return hip_status(rkv::launch_tcond_modulate(
      cfg->num_layers, cfg->num_streams, hidden, tc->num_conds,
      (cfg->flags & RKV_F_OUT_F32) != 0, d_mod, d_stream_cond, d_out,
      static_cast<hipStream_t>(hip_stream)));
}

int rkv_decode_step_pipelined_tcond(const rkv_cfg* cfg, const rkv_tcond_cfg* tc,
                                    const float* d_mod, const int32_t* d_stream_cond,
                                    rkv_stream_state* d_state, const rkv_step_plan* d_plan,
                                    rkv_step_plan* d_plan_next, const rkv_kv_view* kv,
                                    const void* q, const void* k_new, const void* v_new,
                                    void* out, void* workspace, size_t workspace_bytes,
                                    void* hip_stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (cfg->mode == RKV_MODE_ENC_CHUNK) return RKV_EINVAL;
  if ((rc = check_tcond(tc))) return rc;
  if (tc->num_layers != cfg->num_layers || tc->hidden != cfg->num_q_heads * cfg->head_dim)
    return RKV_EINVAL;
  if (!d_stream_cond) return RKV_EINVAL;
  if ((rc = check_ptr(d_mod))) return rc;
  return attention(cfg, rkv::kDecodeFused, d_plan, kv, q, k_new, v_new, out, workspace,
                   workspace_bytes, hip_stream, d_state, d_plan_next, nullptr, 0, d_mod,
                   d_stream_cond, tc->num_conds);
}
