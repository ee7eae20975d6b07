// Cache updates: RoPE-on-append, in-place exact re-base, compaction move.

#include "rkv_device.h"
#include "rkv_internal.h"

namespace rkv {
namespace {

__device__ __forceinline__ void item_coords(int item, int H, int S, int& l, int& s, int& g) {
  g = item % H;
  s = (item / H) % S;
  l = item / (H * S);
}

// ---------------------------------------------------------------------------
// Append (voxtral.c explainer, section 二: K is stored with its rotation baked
// in).  One wave per (layer, stream, kv head, new row); lane i owns rotary
// pair i (elements i and i + d/2) and V elements 2i, 2i+1.
// ---------------------------------------------------------------------------
template <int D, bool COMP, bool ENC, typename SF>
__global__ __launch_bounds__(64) void append_kernel(const rkv_step_plan* __restrict__ plan,
                                                    RingArgs ring,
                                                    const uint16_t* __restrict__ knew,
                                                    const uint16_t* __restrict__ vnew, int S,
                                                    int H, int F) {
  constexpr int HALF = D / 2;
  int l, s, g;
  item_coords(blockIdx.x, H, S, l, s, g);
  const int j = blockIdx.y;
  const rkv_step_plan* P = plan + s;
  if (j >= P->new_rows) return;
  const int slot = (P->slot + j) % P->cap;
  if (slot >= ring.slots) return;  // state capacity beyond the allocated rows
  const int64_t in_off =
      ENC ? ((((int64_t)l * S + s) * F + j) * H + g) * D : (((int64_t)l * S + s) * H + g) * D;
  const int64_t row = (int64_t)l * ring.ls + (int64_t)s * ring.ss + (int64_t)g * ring.hs +
                      (int64_t)slot * ring.rs;
  const int i = threadIdx.x;
  if (i < HALF) {
    const double x1 = bf2f(knew[in_off + i]);
    const double x2 = bf2f(knew[in_off + i + HALF]);
    double y1, y2;
    rotate_pair64(x1, x2, P->rope_new[j][0][i], P->rope_new[j][1][i], y1, y2);
    const uint32_t h1 = SF::from_f64(y1), h2 = SF::from_f64(y2);
    ring.k[row + i] = (uint16_t)h1;
    ring.k[row + i + HALF] = (uint16_t)h2;
    if (COMP) {
      ring.klo[row + i] = (uint16_t)SF::from_f64(y1 - (double)SF::to_f(h1));
      ring.klo[row + i + HALF] = (uint16_t)SF::from_f64(y2 - (double)SF::to_f(h2));
    }
    const uint32_t vv = *reinterpret_cast<const uint32_t*>(vnew + in_off + 2 * i);
    *reinterpret_cast<uint32_t*>(ring.v + row + 2 * i) = SF::from_bf16x2(vv);
  }
}

// ---------------------------------------------------------------------------
// Exact re-base (Audio8 explainer, "Rolling KV Cache 三步拆解" step 2): every
// retained K row is rotated by R(-D) in place (float32 with hi/lo tables and
// exact product errors, rounded to nearest in the storage format: within 1
// ulp of the correctly rounded rotation; the same arithmetic as the fused
// decode step).
// One block per (layer, stream, head) item; a thread owns 8 rotary pairs of a
// row (16 bytes from each half) and walks the item's rows.
// ---------------------------------------------------------------------------
template <int D, bool COMP, typename SF>
__global__ __launch_bounds__(256) void rebase_kernel(const rkv_step_plan* __restrict__ plan,
                                                     RingArgs ring, int S, int H) {
  constexpr int HALF = D / 2;
  constexpr int TPR = HALF / 8;       // threads per row
  constexpr int RPB = 256 / TPR;      // rows per pass of the block
  int l, s, g;
  item_coords(blockIdx.x, H, S, l, s, g);
  const rkv_step_plan* P = plan + s;
  if (P->rebase_delta == 0) return;   // most steps: the whole item is untouched
  const int c = threadIdx.x % TPR;
  const int n_valid = P->n_valid < ring.slots ? P->n_valid : ring.slots;
  const int skip = P->slot;
  f32x4 tab[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    tab[e] = rebase_table_entry(P->rope_delta[0][8 * c + e], P->rope_delta[1][8 * c + e]);
  const int64_t base = (int64_t)l * ring.ls + (int64_t)s * ring.ss + (int64_t)g * ring.hs;
  for (int r = threadIdx.x / TPR; r < n_valid; r += RPB) {
    if (r == skip) continue;
    const int64_t row = base + (int64_t)r * ring.rs;
    uint16_t* k1 = ring.k + row + 8 * c;
    uint16_t* k2 = k1 + HALF;
    u32x4 a = ld16(k1), b = ld16(k2);
    u32x4 la = {0u, 0u, 0u, 0u}, lb = {0u, 0u, 0u, 0u};
    if (COMP) {
      la = ld16(ring.klo + row + 8 * c);
      lb = ld16(ring.klo + row + 8 * c + HALF);
    }
    rebase_chunks_ff<COMP, SF>(a, b, la, lb, [&](int e) { return tab[e]; });
    st16(k1, a);
    st16(k2, b);
    if (COMP) {
      st16(ring.klo + row + 8 * c, la);
      st16(ring.klo + row + 8 * c + HALF, lb);
    }
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
  const dim3 grid(L * S * H, cfg->new_rows);
  const bool comp = (cfg->flags & RKV_F_COMPENSATED) != 0;
  const bool enc = cfg->mode == RKV_MODE_ENC_CHUNK;
  const bool f16 = (cfg->flags & RKV_F_KV_FP16) != 0;
  const int F = cfg->new_rows;
#define RKV_APPEND(DD, CC, EE, SS)                                                             \
  hipLaunchKernelGGL((append_kernel<DD, CC, EE, SS>), grid, dim3(64), 0, stream, plan, ring, \
                     knew, vnew, S, H, F)
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
  const dim3 grid(L * S * H);
#define RKV_REBASE(DD, CC, SS) \
  hipLaunchKernelGGL((rebase_kernel<DD, CC, SS>), grid, dim3(256), 0, stream, plan, ring, S, H)
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
