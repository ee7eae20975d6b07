// Cache updates: RoPE-on-append, in-place exact re-base, compaction move.

#include "rkv_device.h"
#include "rkv_internal.h"
#include "rkv_update.h"

namespace rkv {
namespace {

__device__ __forceinline__ void item_coords(int item, int H, int S, int& l, int& s, int& g) {
  g = item % H;
  s = (item / H) % S;
  l = item / (H * S);
}

// ---------------------------------------------------------------------------
// Append (voxtral.c explainer, section 二: K is stored with its rotation baked
// in).  A unit is one new row of one (layer, stream, kv head) item; TPR = d/16
// lanes share it, lane q owning rotary pairs 8q .. 8q+7 (16 bytes from each
// half of the K row) and 32 bytes of the V row, so every access is a 16-byte
// vector and a 256-thread block writes 256 / TPR rows.
// ---------------------------------------------------------------------------
template <int D, bool COMP, bool ENC, typename SF>
__device__ __forceinline__ void append_unit(const rkv_step_plan* __restrict__ plan,
                                            const RingArgs& ring,
                                            const uint16_t* __restrict__ knew,
                                            const uint16_t* __restrict__ vnew, int S, int H,
                                            int F, int unit, int q) {
  constexpr int HALF = D / 2;
  const int item = unit / F, j = unit - item * F;
  int l, s, g;
  item_coords(item, H, S, l, s, g);
  const rkv_step_plan* P = plan + s;
  if (j >= P->new_rows) return;
  const int slot = (P->slot + j) % P->cap;
  // The host rejects rings with fewer slots than any stream's capacity; this
  // only keeps a corrupted plan from writing outside the ring.
  if (slot >= ring.slots) return;
  const int64_t in_off =
      ENC ? ((((int64_t)l * S + s) * F + j) * H + g) * D : (((int64_t)l * S + s) * H + g) * D;
  const int64_t row = (int64_t)l * ring.ls + (int64_t)s * ring.ss + (int64_t)g * ring.hs +
                      (int64_t)slot * ring.rs;
  const u32x4 x1 = ld16(knew + in_off + 8 * q), x2 = ld16(knew + in_off + HALF + 8 * q);
  const u32x4 v0 = ld16(vnew + in_off + 16 * q), v1 = ld16(vnew + in_off + 16 * q + 8);
  u32x4 h1, h2, lo1, lo2;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    uint32_t a[2], b[2], la[2], lb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = 8 * q + e + u;
      double y1, y2;
      rotate_pair64(bf2f(elem8(x1, e + u)), bf2f(elem8(x2, e + u)), P->rope_new[j][0][i],
                    P->rope_new[j][1][i], y1, y2);
      a[u] = SF::from_f64(y1);
      b[u] = SF::from_f64(y2);
      if (COMP) {
        la[u] = SF::from_f64(y1 - (double)SF::to_f(a[u]));
        lb[u] = SF::from_f64(y2 - (double)SF::to_f(b[u]));
      }
    }
    h1[e >> 1] = a[0] | (a[1] << 16);
    h2[e >> 1] = b[0] | (b[1] << 16);
    if (COMP) {
      lo1[e >> 1] = la[0] | (la[1] << 16);
      lo2[e >> 1] = lb[0] | (lb[1] << 16);
    }
  }
  st16(ring.k + row + 8 * q, h1);
  st16(ring.k + row + HALF + 8 * q, h2);
  if (COMP) {
    st16(ring.klo + row + 8 * q, lo1);
    st16(ring.klo + row + HALF + 8 * q, lo2);
  }
  u32x4 w0, w1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    w0[e] = SF::from_bf16x2(v0[e]);
    w1[e] = SF::from_bf16x2(v1[e]);
  }
  st16(ring.v + row + 16 * q, w0);
  st16(ring.v + row + 16 * q + 8, w1);
}

template <int D, bool COMP, bool ENC, typename SF>
__global__ __launch_bounds__(256) void append_kernel(const rkv_step_plan* __restrict__ plan,
                                                     RingArgs ring,
                                                     const uint16_t* __restrict__ knew,
                                                     const uint16_t* __restrict__ vnew, int S,
                                                     int H, int F, int units) {
  constexpr int TPR = D / 16;         // lanes per row
  const int unit = blockIdx.x * (256 / TPR) + (int)threadIdx.x / TPR;
  if (unit < units)
    append_unit<D, COMP, ENC, SF>(plan, ring, knew, vnew, S, H, F, unit, threadIdx.x % TPR);
}

// ---------------------------------------------------------------------------
// Exact re-base (Audio8 explainer, "Rolling KV Cache 三步拆解" step 2): every
// retained K row is rotated by R(-D) in place (float32 with hi/lo tables and
// exact product errors, rounded to nearest in the storage format: within 1
// ulp of the correctly rounded rotation; the same arithmetic as the fused
// decode step).
// In most steps only the streams whose base moves have work (with staggered
// starts, a few per cent of them, at random places in the grid).  A grid of
// one block per item would sweep mostly empty blocks through the CUs and
// start the last re-basing items only at the end of that sweep, so instead a
// fixed grid of kRebaseBlocks blocks (one resident round) each lists the
// moving streams -- one plan read per stream, a ballot per 64 streams, the
// list compacted in LDS -- and strides over the work units (moving stream,
// layer, head, quarter of the rows).  In a unit a thread owns 8 rotary pairs
// of a row (16 bytes from each half) and walks the rows NB at a time,
// software-pipelined: the loads of the next batch are issued before this
// batch is rotated and stored (the vector memory counter covers stores as
// well as loads, so loads issued after a batch's stores would make the wait
// for them include those stores' acknowledgements).
// ---------------------------------------------------------------------------
constexpr int kRebaseBlocks = 768;       // 256 CUs x 3 resident blocks
constexpr int kRebaseSplit = 4;          // row ranges per item
constexpr int kRebaseListMax = 8192;     // streams listed per pass

template <int D, bool COMP, typename SF>
__device__ __forceinline__ void rebase_rows(const rkv_step_plan* __restrict__ P,
                                            const RingArgs& ring, int l, int s, int g,
                                            int split) {
  constexpr int HALF = D / 2;
  constexpr int TPR = HALF / 8;       // threads per row
  constexpr int RPB = 256 / TPR;      // rows per pass of the block
  constexpr int NB = COMP ? 2 : 4;    // rows per thread per batch
  constexpr int STEP = RPB * NB;      // rows per batch of the block
  const int c = threadIdx.x % TPR;
  const int n_valid = P->n_valid < ring.slots ? P->n_valid : ring.slots;
  const int chunk = (n_valid + kRebaseSplit - 1) / kRebaseSplit;
  const int r_begin = split * chunk;
  const int r_end = min(n_valid, r_begin + chunk);
  if (r_begin >= r_end) return;
  const int skip = P->slot;
  f32x4 tab[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    tab[e] = rebase_table_entry(P->rope_delta[0][8 * c + e], P->rope_delta[1][8 * c + e]);
  const int64_t base =
      (int64_t)l * ring.ls + (int64_t)s * ring.ss + (int64_t)g * ring.hs + 8 * c;
  u32x4 ka[2][NB], kb[2][NB], la[2][NB], lb[2][NB];
  auto load = [&](int buf, int r0) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int r = r0 + j * RPB;
      if (r < r_end && r != skip) {
        const int64_t row = base + (int64_t)r * ring.rs;
        ka[buf][j] = ld16(ring.k + row);
        kb[buf][j] = ld16(ring.k + row + HALF);
        if (COMP) {
          la[buf][j] = ld16(ring.klo + row);
          lb[buf][j] = ld16(ring.klo + row + HALF);
        } else {
          la[buf][j] = lb[buf][j] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };
  auto finish = [&](int buf, int r0) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int r = r0 + j * RPB;
      if (r < r_end && r != skip) {
        const int64_t row = base + (int64_t)r * ring.rs;
        rebase_chunks_ff<COMP, SF>(ka[buf][j], kb[buf][j], la[buf][j], lb[buf][j],
                                   [&](int e) { return tab[e]; });
        st16(ring.k + row, ka[buf][j]);
        st16(ring.k + row + HALF, kb[buf][j]);
        if (COMP) {
          st16(ring.klo + row, la[buf][j]);
          st16(ring.klo + row + HALF, lb[buf][j]);
        }
      }
    }
  };
  int r0 = r_begin + (int)threadIdx.x / TPR;
  load(0, r0);
  for (; r0 < r_end; r0 += 2 * STEP) {
    load(1, r0 + STEP);
    finish(0, r0);
    load(0, r0 + 2 * STEP);
    finish(1, r0 + STEP);
  }
}

// Lists, in LDS, the streams of [s0, s0 + n) whose base moves this step (one
// plan read per stream, a ballot per 64) and returns how many; every thread
// of the block calls it.
struct MovingList {
  static constexpr int kChunks = kRebaseListMax / 64;
  uint16_t stream[kRebaseListMax];
  uint64_t mask[kChunks];
  int offset[kChunks + 1];
};

__device__ int list_moving(const rkv_step_plan* __restrict__ plan, int s0, int n,
                           MovingList& ml) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int chunks = (n + 63) / 64;
  for (int k = wave; k < chunks; k += 4) {
    const int s = s0 + 64 * k + lane;
    const uint64_t m = __ballot(64 * k + lane < n && plan[s].rebase_delta != 0);
    if (lane == 0) ml.mask[k] = m;
  }
  __syncthreads();
  if (t == 0) {
    int acc = 0;
    for (int k = 0; k < chunks; ++k) {
      ml.offset[k] = acc;
      acc += __popcll(ml.mask[k]);
    }
    ml.offset[chunks] = acc;
  }
  __syncthreads();
  for (int k = wave; k < chunks; k += 4) {
    const uint64_t m = ml.mask[k];
    if ((m >> lane) & 1u)
      ml.stream[ml.offset[k] + __popcll(m & ((1ull << lane) - 1ull))] = (uint16_t)(64 * k + lane);
  }
  __syncthreads();
  return ml.offset[chunks];
}

// The re-base units of all moving streams, strided over the grid.
template <int D, bool COMP, typename SF>
__device__ __forceinline__ void rebase_moving(const rkv_step_plan* __restrict__ plan,
                                              const RingArgs& ring, int S, int H, int L,
                                              MovingList& ml) {
  for (int s0 = 0; s0 < S; s0 += kRebaseListMax) {
    const int moving = list_moving(plan, s0, min(S - s0, kRebaseListMax), ml);
    const int64_t units = (int64_t)moving * L * H * kRebaseSplit;
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
      int64_t v = u;
      const int split = (int)(v % kRebaseSplit);
      v /= kRebaseSplit;
      const int g = (int)(v % H);
      v /= H;
      const int l = (int)(v % L);
      const int s = s0 + ml.stream[v / L];
      rebase_rows<D, COMP, SF>(plan + s, ring, l, s, g, split);
    }
    __syncthreads();     // the list is rebuilt for the next pass
  }
}

template <int D, bool COMP, typename SF>
__global__ __launch_bounds__(256) void rebase_kernel(const rkv_step_plan* __restrict__ plan,
                                                     RingArgs ring, int S, int H, int L) {
  __shared__ MovingList ml;
  rebase_moving<D, COMP, SF>(plan, ring, S, H, L, ml);
}

// Re-base and append of one step in one launch: the re-base never touches the
// new row's slot and the append writes only that slot, so the two sets of
// units are independent; the appends are strided over the grid after the
// re-base units.
template <int D, bool COMP, bool ENC, typename SF>
__global__ __launch_bounds__(256) void update_kernel(const rkv_step_plan* __restrict__ plan,
                                                     RingArgs ring,
                                                     const uint16_t* __restrict__ knew,
                                                     const uint16_t* __restrict__ vnew, int S,
                                                     int H, int L, int F) {
  __shared__ MovingList ml;
  if (!ENC) rebase_moving<D, COMP, SF>(plan, ring, S, H, L, ml);
  constexpr int TPR = D / 16;         // lanes per appended row
  constexpr int UPB = 256 / TPR;      // rows per pass of the block
  const int units = L * S * H * F;
  for (int u0 = blockIdx.x * UPB; u0 < units; u0 += gridDim.x * UPB) {
    const int unit = u0 + (int)threadIdx.x / TPR;
    if (unit < units)
      append_unit<D, COMP, ENC, SF>(plan, ring, knew, vnew, S, H, F, unit, threadIdx.x % TPR);
  }
}

// ---------------------------------------------------------------------------
// Compaction move (voxtral.c explainer, section 二): rows [drop, drop + W) go
// to [0, W) in row order.  The ranges overlap, so the rows are moved front to
// back in batches of at most `drop` rows: a batch reads rows that no earlier
// batch wrote and writes rows that only earlier batches read.  One block moves
// the K (or V) rows of one item, whole rows at a time; the barrier after each
// batch's stores (which need its loads' data) makes every read of the batch
// complete before the next batch writes.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void compact_kernel(const rkv_step_plan* __restrict__ plan,
                                                      RingArgs ring, int S, int H) {
  constexpr int TPR = D / 8;            // threads per row (16 bytes each)
  constexpr int RPR = 256 / TPR;        // rows per load instruction of the block
  constexpr int NB = 8;                 // loads in flight per thread
  int l, s, g;
  item_coords(blockIdx.x, H, S, l, s, g);
  const rkv_step_plan* P = plan + s;
  const int drop = P->compact_drop;
  // (cap > slots cannot pass the host checks; kept as a bound on a corrupted plan)
  if (drop == 0 || P->cap > ring.slots) return;
  const int rows = P->window;
  uint16_t* base = (blockIdx.y == 0 ? ring.k : ring.v) + (int64_t)l * ring.ls +
                   (int64_t)s * ring.ss + (int64_t)g * ring.hs;
  const int col = (threadIdx.x % TPR) * 8;
  const int ro = threadIdx.x / TPR;
  const int batch = RPR * NB < drop ? RPR * NB : drop;
  for (int r0 = 0; r0 < rows; r0 += batch) {
    const int rend = r0 + batch < rows ? r0 + batch : rows;
    u32x4 buf[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int r = r0 + ro + RPR * k;
      if (r < rend) buf[k] = ld16(base + (int64_t)(r + drop) * ring.rs + col);
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int r = r0 + ro + RPR * k;
      if (r < rend) st16(base + (int64_t)r * ring.rs + col, buf[k]);
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_append(const rkv_cfg* cfg, const rkv_step_plan* plan, const RingArgs& ring,
                         const uint16_t* knew, const uint16_t* vnew, hipStream_t stream) {
  const int S = cfg->num_streams, H = cfg->num_kv_heads, L = cfg->num_layers;
  const bool comp = (cfg->flags & RKV_F_COMPENSATED) != 0;
  const bool enc = cfg->mode == RKV_MODE_ENC_CHUNK;
  const bool f16 = (cfg->flags & RKV_F_KV_FP16) != 0;
  const int F = cfg->new_rows;
  const int units = L * S * H * F;
  const int per_block = 256 / (cfg->head_dim / 16);
  const dim3 grid((units + per_block - 1) / per_block);
#define RKV_APPEND(DD, CC, EE, SS)                                                              \
  hipLaunchKernelGGL((append_kernel<DD, CC, EE, SS>), grid, dim3(256), 0, stream, plan, ring, \
                     knew, vnew, S, H, F, units)
#define RKV_APPEND_D(DD)                                 \
  if (enc) RKV_APPEND(DD, false, true, StoreBf16);       \
  else if (comp && f16) RKV_APPEND(DD, true, false, StoreF16);  \
  else if (comp) RKV_APPEND(DD, true, false, StoreBf16); \
  else if (f16) RKV_APPEND(DD, false, false, StoreF16);  \
  else RKV_APPEND(DD, false, false, StoreBf16)
  if (cfg->head_dim == 128) {
    RKV_APPEND_D(128);
  } else {
    RKV_APPEND_D(64);
  }
#undef RKV_APPEND_D
#undef RKV_APPEND
  return hipGetLastError();
}

hipError_t launch_rebase(const rkv_cfg* cfg, const rkv_step_plan* plan, const RingArgs& ring,
                         hipStream_t stream) {
  const int S = cfg->num_streams, H = cfg->num_kv_heads, L = cfg->num_layers;
  const bool comp = (cfg->flags & RKV_F_COMPENSATED) != 0;
  const bool f16 = (cfg->flags & RKV_F_KV_FP16) != 0;
  const dim3 grid(kRebaseBlocks);
#define RKV_REBASE(DD, CC, SS)                                                             \
  hipLaunchKernelGGL((rebase_kernel<DD, CC, SS>), grid, dim3(256), 0, stream, plan, ring, S, H, \
                     L)
#define RKV_REBASE_D(DD)                                    \
  if (comp && f16) RKV_REBASE(DD, true, StoreF16);          \
  else if (comp) RKV_REBASE(DD, true, StoreBf16);           \
  else if (f16) RKV_REBASE(DD, false, StoreF16);            \
  else RKV_REBASE(DD, false, StoreBf16)
  if (cfg->head_dim == 128) {
    RKV_REBASE_D(128);
  } else {
    RKV_REBASE_D(64);
  }
#undef RKV_REBASE_D
#undef RKV_REBASE
  return hipGetLastError();
}

hipError_t launch_update(const rkv_cfg* cfg, const rkv_step_plan* plan, const RingArgs& ring,
                         const uint16_t* knew, const uint16_t* vnew, hipStream_t stream) {
  const int S = cfg->num_streams, H = cfg->num_kv_heads, L = cfg->num_layers;
  const bool comp = (cfg->flags & RKV_F_COMPENSATED) != 0;
  const bool enc = cfg->mode == RKV_MODE_ENC_CHUNK;
  const bool f16 = (cfg->flags & RKV_F_KV_FP16) != 0;
  const int F = cfg->new_rows;
  const dim3 grid(kRebaseBlocks);
#define RKV_UPDATE(DD, CC, EE, SS)                                                              \
  hipLaunchKernelGGL((update_kernel<DD, CC, EE, SS>), grid, dim3(256), 0, stream, plan, ring, \
                     knew, vnew, S, H, L, F)
#define RKV_UPDATE_D(DD)                                        \
  if (enc) RKV_UPDATE(DD, false, true, StoreBf16);              \
  else if (comp && f16) RKV_UPDATE(DD, true, false, StoreF16);  \
  else if (comp) RKV_UPDATE(DD, true, false, StoreBf16);        \
  else if (f16) RKV_UPDATE(DD, false, false, StoreF16);         \
  else RKV_UPDATE(DD, false, false, StoreBf16)
  if (cfg->head_dim == 128) {
    RKV_UPDATE_D(128);
  } else {
    RKV_UPDATE_D(64);
  }
#undef RKV_UPDATE_D
#undef RKV_UPDATE
  return hipGetLastError();
}

hipError_t launch_compact(const rkv_cfg* cfg, const rkv_step_plan* plan, const RingArgs& ring,
                          hipStream_t stream) {
  const int S = cfg->num_streams, H = cfg->num_kv_heads, L = cfg->num_layers;
  const dim3 grid(L * S * H, 2);
  if (cfg->head_dim == 128)
    hipLaunchKernelGGL((compact_kernel<128>), grid, dim3(256), 0, stream, plan, ring, S, H);
  else
    hipLaunchKernelGGL((compact_kernel<64>), grid, dim3(256), 0, stream, plan, ring, S, H);
  return hipGetLastError();
}

}  // namespace rkv
