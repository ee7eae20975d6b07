// Windowed attention over the rolling cache on gfx950 matrix cores.
//
// One workgroup of NW waves handles one (layer, stream, kv head) item -- or
// one split of its key range.  The waves take 16-key tiles in turn, each
// keeping two tiles in registers (one computing, one loading), and merge their
// partial softmax states through LDS at the end.  With the whole chip
// streaming, a workgroup's life is set by its share of its CU's bandwidth, so
// more waves per item (shorter lives) mainly shortens the drain at the end of
// the launch, when too few workgroups remain to keep HBM busy.  The G query
// vectors that share the KV head (the 8 query heads of a GQA group, or the F
// frames of an encoder chunk) form the N side of the matrix-core products:
//
//   scores  S[key][col] = K[key][:] . Qt[:][col]   v_mfma_f32_16x16x32_bf16
//   output  O[d][col]  += Vt[d][key] . P[key][col]  v_mfma_f32_16x16x16_bf16
//
// Only 8 of the 16 columns are query vectors, so the other 8 carry the
// bfloat16 rounding residual of the same vectors: column c < 8 holds
// hi = rne(x) and column c + 8 holds lo = rne(x - hi), for the rotated query
// and for the probabilities.  Adding the two columns (a row_ror:8 DPP move)
// gives scores and outputs at about 16-bit operand precision at no extra
// matrix-core work.  K and V are the stored bfloat16 values.
//
// Lane layout (lane = 16*g4 + c).  Score MFMA: A holds K row key0+c, dims
// 32*st + 8*g4 .. +7; B holds query column c, the same dims; the result holds
// keys key0 + 4*g4 + r (r < 4) of column c -- exactly the B layout of the
// 16x16x16 probability MFMA (k = 4*g4 .. 4*g4+3).  V rows key0 + 4*g4 + j
// (j < 4) are loaded row-contiguously (lane reads dims CW*c .. CW*c+CW-1, so
// each load instruction covers four whole rows) and transposed in registers
// (v_perm) into the A operand (row c <-> dim CW*c + e for product e).  Output
// lane (g4, c < 8) ends with dims [4*CW*g4, 4*CW*g4 + 4*CW) of column c.
//
// The rotated query is built once per workgroup (all waves share the rotary
// pairs) and shared through LDS.  Each wave requests its query chunks, rotary
// tables and new row first and its first two tiles right after them (vector
// loads complete in issue order), so set-up waits only for the small loads
// and runs with two tiles in flight.  Softmax is online with a lazily moved
// maximum: probabilities use the running maximum m until a tile's maximum
// exceeds it by more than 2^8 (log2 units), so accumulator rescaling is rare.
//
// The fused kinds also update the cache in the same launch, with results
// identical to running rkv_roll_rebase, rkv_append and the read-only kind in
// turn.  Decoder: during set-up the waves rotate the new K row from k_new in
// float64 (the rotary pairs split over all waves), write K and V to the ring and leave
// both in LDS, from where the wave whose tile holds the new slot patches them
// into its registers (its tile may have been read before the write).  In
// REBASE mode, when the plan's delta D > 0, each wave re-bases the rows of its
// tiles in registers as they arrive (R(-D) in float32 with hi/lo tables and
// exact product errors, rounded to bfloat16: the arithmetic of rkv_roll_rebase)
// and writes them back, so K is read once.
// Encoder: each wave writes the new frames that fall in its own tiles before
// reading them.

#include <stddef.h>

#include <type_traits>

#include "rkv_device.h"
#include "rkv_internal.h"

namespace rkv {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// The two matrix-core products in the cache's storage format SF (bfloat16,
// or binary16 for the fp16 cache variant); float32 accumulation either way.
template <typename SF>
struct Mfma;
template <>
struct Mfma<StoreBf16> {
  static __device__ __forceinline__ f32x4 scores(const u32x4& a, const u32x4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(const u32x2& a, const u32x2& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  }
};
template <>
struct Mfma<StoreF16> {
  static __device__ __forceinline__ f32x4 scores(const u32x4& a, const u32x4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(const u32x2& a, const u32x2& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
};

__device__ __forceinline__ float dpp_ror8(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// low / high bfloat16 halves of two words, packed: {a.lo, b.lo} or {a.hi, b.hi}
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// A lane's V chunk of one row (CW elements; 16 lanes cover a row, so each
// load instruction reads whole lines: V rows are streamed, read once a launch).
template <int CW>
struct VChunk;
template <>
struct VChunk<8> {
  typedef u32x4 T;
  template <typename SF>
  static __device__ __forceinline__ T from_input(const T& w) {
    return T{SF::from_bf16x2(w[0]), SF::from_bf16x2(w[1]), SF::from_bf16x2(w[2]),
             SF::from_bf16x2(w[3])};
  }
  static __device__ __forceinline__ T load(const uint16_t* p) { return ld16_stream(p); }
  static __device__ __forceinline__ void store(uint16_t* p, const T& w) { st16(p, w); }
  static __device__ __forceinline__ T zero() { return u32x4{0u, 0u, 0u, 0u}; }
};
template <>
struct VChunk<4> {
  typedef u32x2 T;
  template <typename SF>
  static __device__ __forceinline__ T from_input(const T& w) {
    return T{SF::from_bf16x2(w[0]), SF::from_bf16x2(w[1])};
  }
  static __device__ __forceinline__ T load(const uint16_t* p) { return ld8_stream(p); }
  static __device__ __forceinline__ void store(uint16_t* p, const T& w) { st8(p, w); }
  static __device__ __forceinline__ T zero() { return u32x2{0u, 0u}; }
};

constexpr float kLazyMax = 8.0f;  // rescale only when the max grows by > 2^8

// Waves per SIMD the register allocation targets: 3, the fastest measured for
// both head sizes (d = 64 would fit 4, which ran ~1 % slower: a fuller
// memory queue lengthens every load's wait), or 2 where the compensated
// re-base keeps two more K arrays live at d = 128.
template <int D, bool COMP>
struct Occupancy {
  static constexpr int waves = D == 128 && COMP ? 2 : 3;
};

// Merge of an item's split partials by the last split to finish, in the
// attention launch:  out = sum_j 2^(m_j - M) num_j / sum_j 2^(m_j - M) l_j,
// M = max_j m_j, the sums taken over the splits in order -- the arithmetic of
// combine_kernel, so the two merges give the same bits.  Thread `tid` of NT
// takes the output quads tid, tid + NT, ... (head hh, dims dd .. dd + 3); the
// partials are read with device-scope loads (pb covers the item's partials),
// up to 8 splits in flight.  `base` is the output offset of head 0 and
// `hstride` the distance between heads.
template <int D, int NT>
__device__ __forceinline__ void merge_partials(__amdgpu_buffer_rsrc_t pb, const AttnArgs& a,
                                               int64_t base, int64_t hstride, int tid,
                                               const float* tg) {
  const int ns = a.nsplit;
  const int pf = (int)partial_floats(D);
  const int nq = a.G * (D / 4);
  for (int qd = tid; qd < nq; qd += NT) {
    const int hh = qd / (D / 4);
    const int dd = 4 * (qd - hh * (D / 4));
    float m8[8], l8[8];
    f32x4 v8[8];
    auto fetch = [&](int j0) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u < ns ? j0 + u : ns - 1;  // clamped: read, never used
        m8[u] = ld_dev(pb, 4 * (j * pf + hh));
        l8[u] = ld_dev(pb, 4 * (j * pf + 8 + hh));
        v8[u] = ld_dev4(pb, 4 * (j * pf + 16 + hh * D + dd));
      }
    };
    fetch(0);
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u < ns) M = fmaxf(M, m8[u]);
    for (int j = 8; j < ns; ++j) M = fmaxf(M, ld_dev(pb, 4 * (j * pf + hh)));
    float den = 0.f;
    f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < ns; j0 += 8) {
      if (j0 > 0) fetch(j0);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (j0 + u < ns) {
          const float f = (M == -INFINITY || m8[u] == -INFINITY) ? 0.f : fast_exp2(m8[u] - M);
          den += f * l8[u];
          num += f * v8[u];
        }
      }
    }
    float o4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) o4[k] = den > 0.f ? num[k] / den : 0.f;
    const int64_t off = base + hh * hstride + dd;
    // delay conditioning of the stored value (tg: gamma of head 0, beta a
    // hidden width later; decoder only)
    if (tg) {
      const int hidden = a.Hkv * a.G * D;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = hh * D + dd + k;
        const float x = a.out_f32 ? o4[k] : bf2f(f2bf(o4[k]));
        o4[k] = fmaf(x, 1.0f + tg[i], tg[hidden + i]);
      }
    }
    if (a.out_f32)
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + off) =
          f32x4{o4[0], o4[1], o4[2], o4[3]};
    else
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + off) =
          u32x2{f2bf(o4[0]) | (f2bf(o4[1]) << 16), f2bf(o4[2]) | (f2bf(o4[3]) << 16)};
  }
}

template <int D, int NW, int KIND, bool COMP, typename SF, bool KL>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(Occupancy<D, COMP>::waves)))
void attn_kernel(AttnArgs args) {
  constexpr int KS = D / 32;    // k-steps of the score MFMA (32 dims each)
  constexpr int KH = KS / 2;    // k-steps of the first half (pair partner is st + KH)
  constexpr int CW = D / 16;    // V elements per lane per row = probability MFMAs per tile
  constexpr int TK = 16;        // keys per tile
  typedef VChunk<CW> VC;
  typedef typename VC::T VT;

  __shared__ u32x4 sm_q[KS][64];
  __shared__ u32x4 sm_newk[KS][4];   // decoder: the appended K row, chunk (st, g4)
  __shared__ VT sm_newv[16];         // decoder: the appended V row, chunk c
  __shared__ float sm_m[NW][8];
  __shared__ float sm_l[NW][8];
  __shared__ f32x4 sm_o[NW > 1 ? NW - 1 : 1][CW][32];  // [wave-1][e][8*g4 + c], c < 8
  __shared__ f32x4 sm_dt[D / 2];  // re-base: hi/lo float32 of cos(D theta_i), -sin(D theta_i)

  // Every argument but the theta table of the plan-advance blocks, copied
  // up front and pinned in scalar registers, so the argument loads are issued
  // together and awaited once (fetched at each first use, they cost a round
  // trip to the argument buffer apiece).
  AttnArgs a;
  a.plan = args.plan;
  a.ring = args.ring;
  a.q = args.q;
  a.knew = args.knew;
  a.vnew = args.vnew;
  a.out = args.out;
  a.ws = args.ws;
  a.tickets = args.tickets;
  a.S = args.S;
  a.L = args.L;
  a.Hkv = args.Hkv;
  a.G = args.G;
  a.F = args.F;
  a.nsplit = args.nsplit;
  a.out_f32 = args.out_f32;
  a.scale_log2 = args.scale_log2;
  a.adv_state = args.adv_state;
  a.adv_plan = args.adv_plan;
  a.adv_mode = args.adv_mode;
  a.adv_dc = args.adv_dc;
  a.adv_F = args.adv_F;
  a.adv_half = args.adv_half;
  a.pull = args.pull;
  a.pull_bytes = args.pull_bytes;
  a.pull_blocks = args.pull_blocks;
  a.tc_mod = args.tc_mod;
  a.tc_cond = args.tc_cond;
  a.tc_conds = args.tc_conds;
  asm volatile("" : : "s"(a.plan), "s"(a.ring.k), "s"(a.ring.v), "s"(a.ring.klo), "s"(a.ring.ls),
               "s"(a.ring.ss), "s"(a.ring.hs), "s"(a.ring.rs), "s"(a.ring.slots));
  asm volatile("" : : "s"(a.q), "s"(a.knew), "s"(a.vnew), "s"(a.out), "s"(a.ws), "s"(a.S),
               "s"(a.L), "s"(a.Hkv), "s"(a.G), "s"(a.F), "s"(a.nsplit), "s"(a.out_f32),
               "s"(a.scale_log2), "s"(a.adv_state), "s"(a.tickets));

  // Encoder step: the blocks past the attention grid pull the next products'
  // weights into the cache while the attention drains.
  if (KIND == kEncoderFused && a.pull) {
    const int njobs = a.L * a.S * a.Hkv * a.nsplit;
    if ((int)blockIdx.x >= njobs) {
      pull_into_cache(a.pull, a.pull_bytes, (int)blockIdx.x - njobs, a.pull_blocks,
                      reinterpret_cast<uint16_t*>(&sm_q[0][0]));
      return;
    }
  }
  // Pipelined decode step: the blocks past the attention grid compute the
  // next step's plan, one wave per stream (nothing in this launch reads it).
  if ((KIND == kDecodeFused || KIND == kDecodeRead) && a.adv_state) {
    const int njobs = a.L * a.S * a.Hkv * a.nsplit;
    if ((int)blockIdx.x >= njobs) {
      const int s = ((int)blockIdx.x - njobs) * NW + (int)(threadIdx.x >> 6);
      if (s < a.S)
        advance_stream(a.adv_state, a.adv_plan, s, threadIdx.x & 63, a.adv_mode, a.adv_dc,
                       a.adv_F, a.adv_half, args.adv_theta);
      return;
    }
  }

  const int lane = threadIdx.x & 63;
  // wave index made provably uniform, so tile-index branches are scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15;
  const int g4 = lane >> 4;
  const int col_q = c & 7;       // query vector of this column
  const int part = c >> 3;       // 0: hi, 1: lo residual

  const int split = blockIdx.x % a.nsplit;
  const int item = blockIdx.x / a.nsplit;
  const int g = item % a.Hkv;
  const int s = (item / a.Hkv) % a.S;
  const int l = item / (a.Hkv * a.S);
  const rkv_step_plan* P = a.plan + s;
  // The plan header (t, pos, first_pos, slot, n_valid, rebase_delta, cap,
  // new_rows) is requested with the other set-up loads and read only after
  // the first tiles are requested, so that no load waits for it.
  // (Only words that are used are loaded: a load whose destination holds a
  // dead word makes the next writer of that register wait for it.)
  const char* phb = reinterpret_cast<const char*>(P);
  const u32x4 hd0 = *reinterpret_cast<const u32x4*>(phb);                         // t, pos
  const u32x2 hd1 = *reinterpret_cast<const u32x2*>(phb + offsetof(rkv_step_plan, first_pos));
  const u32x2 hd2 = *reinterpret_cast<const u32x2*>(phb + offsetof(rkv_step_plan, slot));
  const uint32_t hd3 = *reinterpret_cast<const uint32_t*>(phb +
                                                          offsetof(rkv_step_plan, rebase_delta));
  const u32x2 hd4 = *reinterpret_cast<const u32x2*>(phb + offsetof(rkv_step_plan, cap));
  // delay conditioning: the stream's condition, requested with the set-up
  const int tc_c = (KIND != kEncoderFused && a.tc_mod) ? a.tc_cond[s] : -1;

  const int slots = a.ring.slots;
  const int per = (((slots + a.nsplit - 1) / a.nsplit) + TK - 1) & ~(TK - 1);
  const int kb = split * per;

  const int64_t rbase = (int64_t)l * a.ring.ls + (int64_t)s * a.ring.ss + (int64_t)g * a.ring.hs;
  uint16_t* __restrict__ Kp = a.ring.k + rbase;
  uint16_t* __restrict__ Vp = a.ring.v + rbase;
  uint16_t* __restrict__ Lp = COMP ? a.ring.klo + rbase : nullptr;
  const int64_t rs = a.ring.rs;

  // Offsets of query vector j in the [L][S][Hkv*G][D] (decoder) or
  // [L][S][F][H][D] (encoder) inputs and outputs, and of new K/V row j in
  // [L][S][Hkv][D] (decoder) or [L][S][F][H][D] (encoder).
  auto vec_off = [&](int j) -> int64_t {
    if (KIND == kEncoderFused) return ((((int64_t)l * a.S + s) * a.F + j) * a.Hkv + g) * D;
    return ((((int64_t)l * a.S + s) * a.Hkv + g) * a.G + j) * D;
  };
  auto new_off = [&](int j) -> int64_t {
    if (KIND == kEncoderFused) return vec_off(j);
    return (((int64_t)l * a.S + s) * a.Hkv + g) * D;
  };

  // The compensated decoder also carries the K residual chunks of its rows.
  constexpr bool LO = COMP && KIND == kDecodeFused;
  struct Tile {
    u32x4 k[KS];
    VT v[4];
    u32x4 lo[LO ? KS : 1];
  };
  // Rows past `lim` (the last row that may be read) are clamped to it, so a
  // partial tile reads valid data; its masked keys get probability 0.
  auto load_tile = [&](int key0, Tile& T, int lim) {
    const int rk = key0 + c < lim ? key0 + c : lim;
    if (KL) {
      // K in whole 128-byte lines, streamed: load st = 2 ln + h reads line ln
      // of keys key0 + 8 h .. + 7, lane -> key lane & 7, 16-byte chunk
      // 4 ((lane >> 3) & 1) + (lane >> 4) of the line; fix_k() moves the
      // words to the operand layout before the tile is used
      const int kr0 = key0 + (lane & 7);
      const int ch = 4 * ((lane >> 3) & 1) + (lane >> 4);
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const int r = kr0 + 8 * (st & 1) < lim ? kr0 + 8 * (st & 1) : lim;
        T.k[st] = ld16_stream(Kp + r * rs + 64 * (st >> 1) + 8 * ch);
      }
    } else {
#pragma unroll
      for (int st = 0; st < KS; ++st) T.k[st] = ld16(Kp + rk * rs + 32 * st + 8 * g4);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rv0 = key0 + 4 * g4 + j;
      const int rv = rv0 < lim ? rv0 : lim;
      T.v[j] = VC::load(Vp + rv * rs + CW * c);
    }
    if (LO) {
#pragma unroll
      for (int st = 0; st < KS; ++st) T.lo[st] = ld16(Lp + rk * rs + 32 * st + 8 * g4);
    }
  };

  // ---- loads issued before any result is needed ----
  // Order matters: vector loads complete in issue order, so the query and its
  // rotary tables come first (the set-up waits only for them) and the wave's
  // first two tiles after them, so that set-up runs with two tiles in flight.
  // Tiles read here are clamped into the allocation (rows past the valid
  // range are masked in process()).
  //
  // Set-up work (rotated query, decoder's new K row) is split over all waves
  // in units of one 32-bit word of one chunk pair: unit u covers elements
  // 2w, 2w + 1 (w = u / KH) of chunks st and st + KH (st = u % KH) of the
  // lane's 8-element slices; wave v takes units v, v + NW, ...
  constexpr int UNITS = KH * 4;
  constexpr int UPW = (UNITS + NW - 1) / NW;  // units per wave
  const bool qhas = col_q < a.G;
  uint32_t qw1[UPW], qw2[UPW];
  // cos/sin of the unit's two rotary pairs at the new position (float64: the
  // decoder's new K row uses them as they are, the query in float32)
  double rcs[UPW][2], rsn[UPW][2];
  uint32_t kw1[UPW], kw2[UPW];
  auto unit_st = [&](int k) { return (wave + NW * k) % KH; };
  auto unit_w = [&](int k) { return ((wave + NW * k) / KH) & 3; };
  {
    const uint16_t* qp = a.q + vec_off(qhas ? col_q : 0);
    const int rrow = (KIND == kEncoderFused) ? col_q : 0;
#pragma unroll
    for (int k = 0; k < UPW; ++k) {
      const int st = unit_st(k), w = unit_w(k);
      const int o = 32 * st + 8 * g4 + 2 * w;
      qw1[k] = qhas ? *reinterpret_cast<const uint32_t*>(qp + o) : 0u;
      qw2[k] = qhas ? *reinterpret_cast<const uint32_t*>(qp + o + 32 * KH) : 0u;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        rcs[k][h] = P->rope_new[rrow][0][o + h];
        rsn[k][h] = P->rope_new[rrow][1][o + h];
      }
    }
  }
  // Decoder's new row: the last wave copies V.  K and V are patched into their
  // tile from LDS inside the loop.
  VT vnew_c;
  if (KIND == kDecodeFused) {
    const uint16_t* kn = a.knew + new_off(0);
#pragma unroll
    for (int k = 0; k < UPW; ++k) {
      const int o = 32 * unit_st(k) + 8 * g4 + 2 * unit_w(k);
      kw1[k] = *reinterpret_cast<const uint32_t*>(kn + o);
      kw2[k] = *reinterpret_cast<const uint32_t*>(kn + o + 32 * KH);
    }
    vnew_c = VC::load(a.vnew + new_off(0) + CW * c);
  }
  // The re-base angle's float64 cos/sin (used only when the base moves; wave
  // 0 turns them into the float32 tables), requested with the set-up loads.
  double dt_c = 1.0, dt_s = 0.0;
  if (KIND == kDecodeFused && wave == 0) {
    const int i = lane < D / 2 ? lane : 0;
    dt_c = P->rope_delta[0][i];
    dt_s = P->rope_delta[1][i];
  }
  // keep the tile loads behind the set-up loads in issue order
  __builtin_amdgcn_sched_barrier(0);
  const int first = kb + TK * wave;
  const int kalloc = kb + per < slots ? kb + per : slots;
  Tile tb[2];
  load_tile(first, tb[0], kalloc - 1 > 0 ? kalloc - 1 : 0);
  load_tile(first + TK * NW, tb[1], kalloc - 1 > 0 ? kalloc - 1 : 0);
  // everything above is requested before anything below waits for data
  __builtin_amdgcn_sched_barrier(0);

  // plan header fields (uniform: read from the first lane)
  const int64_t plan_t = ((int64_t)__builtin_amdgcn_readfirstlane(hd0[1]) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane(hd0[0]);
  const int64_t plan_pos = ((int64_t)__builtin_amdgcn_readfirstlane(hd0[3]) << 32) |
                           (uint32_t)__builtin_amdgcn_readfirstlane(hd0[2]);
  const int64_t first_pos = ((int64_t)__builtin_amdgcn_readfirstlane(hd1[1]) << 32) |
                            (uint32_t)__builtin_amdgcn_readfirstlane(hd1[0]);
  const int slot_new = __builtin_amdgcn_readfirstlane(hd2[0]);
  const int plan_n_valid = __builtin_amdgcn_readfirstlane(hd2[1]);
  const int plan_delta = __builtin_amdgcn_readfirstlane(hd3);
  const int cap = __builtin_amdgcn_readfirstlane(hd4[0]);
  const int nnew = __builtin_amdgcn_readfirstlane(hd4[1]);
  static_assert(offsetof(rkv_step_plan, pos) == 8 &&
                    offsetof(rkv_step_plan, n_valid) == offsetof(rkv_step_plan, slot) + 4 &&
                    offsetof(rkv_step_plan, new_rows) == offsetof(rkv_step_plan, cap) + 4,
                "plan header layout");
  // n_valid <= cap <= slots is guaranteed by the host checks; the clamp only
  // bounds the reads of a corrupted plan
  const int n_valid = plan_n_valid < slots ? plan_n_valid : slots;
  const int ke = kb + per < n_valid ? kb + per : n_valid;

#pragma unroll
  for (int k = 0; k < UPW; ++k) {
    if (wave + NW * k >= UNITS) continue;
    const int st = unit_st(k), w = unit_w(k);
    float y1[2], y2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float a1 = bf2f((qw1[k] >> (16 * h)) & 0xffffu);
      const float a2 = bf2f((qw2[k] >> (16 * h)) & 0xffffu);
      const float cq = (float)rcs[k][h], sq = (float)rsn[k][h];
      y1[h] = fmaf(a1, cq, -(a2 * sq));
      y2[h] = fmaf(a1, sq, a2 * cq);
    }
    const uint32_t h1 = SF::cvt2(y1[0], y1[1]);
    const uint32_t h2 = SF::cvt2(y2[0], y2[1]);
    reinterpret_cast<uint32_t*>(&sm_q[st][lane])[w] =
        part ? SF::cvt2(y1[0] - SF::to_f(h1 & 0xffffu), y1[1] - SF::to_f(h1 >> 16)) : h1;
    reinterpret_cast<uint32_t*>(&sm_q[st + KH][lane])[w] =
        part ? SF::cvt2(y2[0] - SF::to_f(h2 & 0xffffu), y2[1] - SF::to_f(h2 >> 16)) : h2;
  }

  // ---- fused-update parameters ----
  const int delta = (KIND == kDecodeFused) ? plan_delta : 0;

  auto new_index = [&](int row) -> int {
    if (KIND == kDecodeFused) return row == slot_new ? 0 : -1;
    const int dj = (row - slot_new + cap) % cap;
    return dj < nnew ? dj : -1;
  };

  // Rotate this lane's K chunks of one row in float64, store them correctly
  // rounded; pairs are chunks (st, st + KH).  src: chunks to rotate (k_new or
  // the stored row); lo: stored residual (compensated re-base); sgn = -1
  // rotates by the negative angle.
  auto rotate_row = [&](const u32x4* src, const u32x4* lo, const double* cs, const double* sn,
                        double sgn, int row, u32x4* kout) {
#pragma unroll
    for (int st = 0; st < KH; ++st) {
      u32x4 w1, w2, r1, r2;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        double y1[2], y2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int e = 2 * w + h;
          const int i = 32 * st + 8 * g4 + e;
          double x1 = bf2f(elem8(src[st], e)), x2 = bf2f(elem8(src[st + KH], e));
          if (COMP && lo) {
            x1 += (double)SF::to_f(elem8(lo[st], e));
            x2 += (double)SF::to_f(elem8(lo[st + KH], e));
          }
          rotate_pair64(x1, x2, cs[i], sgn * sn[i], y1[h], y2[h]);
        }
        w1[w] = SF::cvt2_f64(y1[0], y1[1]);
        w2[w] = SF::cvt2_f64(y2[0], y2[1]);
        if (COMP) {
          r1[w] = SF::cvt2_f64(y1[0] - (double)SF::to_f(w1[w] & 0xffffu),
                               y1[1] - (double)SF::to_f(w1[w] >> 16));
          r2[w] = SF::cvt2_f64(y2[0] - (double)SF::to_f(w2[w] & 0xffffu),
                               y2[1] - (double)SF::to_f(w2[w] >> 16));
        }
      }
      st16(Kp + row * rs + 32 * st + 8 * g4, w1);
      st16(Kp + row * rs + 32 * (st + KH) + 8 * g4, w2);
      if (kout) {
        kout[st] = w1;
        kout[st + KH] = w2;
      }
      if (COMP) {
        st16(Lp + row * rs + 32 * st + 8 * g4, r1);
        st16(Lp + row * rs + 32 * (st + KH) + 8 * g4, r2);
      }
    }
  };

  // Decoder RoPE-on-append: the waves rotate the new K row (float64,
  // correctly rounded) unit by unit, write K and V to the ring and leave both
  // in LDS for the wave whose tile holds the new slot.
  if (KIND == kDecodeFused) {
#pragma unroll
    for (int k = 0; k < UPW; ++k) {
      if (wave + NW * k >= UNITS) continue;
      const int st = unit_st(k), w = unit_w(k);
      double y1[2], y2[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
        rotate_pair64(bf2f((kw1[k] >> (16 * h)) & 0xffffu), bf2f((kw2[k] >> (16 * h)) & 0xffffu),
                      rcs[k][h], rsn[k][h], y1[h], y2[h]);
      const uint32_t w1 = SF::cvt2_f64(y1[0], y1[1]);
      const uint32_t w2 = SF::cvt2_f64(y2[0], y2[1]);
      if (c == 0) {
        reinterpret_cast<uint32_t*>(&sm_newk[st][g4])[w] = w1;
        reinterpret_cast<uint32_t*>(&sm_newk[st + KH][g4])[w] = w2;
      }
      // every split keeps the new row in LDS; split 0 writes it to the ring
      if (c == 0 && split == 0) {
        const int o = 32 * st + 8 * g4 + 2 * w;
        *reinterpret_cast<uint32_t*>(Kp + slot_new * rs + o) = w1;
        *reinterpret_cast<uint32_t*>(Kp + slot_new * rs + o + 32 * KH) = w2;
        if (COMP) {
          *reinterpret_cast<uint32_t*>(Lp + slot_new * rs + o) = SF::cvt2_f64(
              y1[0] - (double)SF::to_f(w1 & 0xffffu), y1[1] - (double)SF::to_f(w1 >> 16));
          *reinterpret_cast<uint32_t*>(Lp + slot_new * rs + o + 32 * KH) = SF::cvt2_f64(
              y2[0] - (double)SF::to_f(w2 & 0xffffu), y2[1] - (double)SF::to_f(w2 >> 16));
        }
      }
    }
    if (wave == NW - 1 && g4 == 0) {
      const VT vs = VC::template from_input<SF>(vnew_c);
      sm_newv[c] = vs;
      if (split == 0) VC::store(Vp + slot_new * rs + CW * c, vs);
    }
  }

  auto key_of = [&](int i) { return first + TK * NW * i; };
  const int ntiles = first < ke ? (ke - first + TK * NW - 1) / (TK * NW) : 0;
  const int lim0 = ke > 0 ? ke - 1 : 0;  // last readable row of the valid range
  // Encoder RoPE-on-append: each wave writes the new frames that fall in its
  // own tiles (float64, correctly rounded) and reads those tiles again.
  if (KIND == kEncoderFused) {
    for (int tt = 0; tt < ntiles; ++tt) {
      const int key0 = key_of(tt);
      const int row = key0 + c;
      if (row < ke) {
        const int jn = new_index(row);
        if (jn >= 0) {
          u32x4 src[KS];
          const uint16_t* kn = a.knew + new_off(jn);
#pragma unroll
          for (int st = 0; st < KS; ++st) src[st] = ld16(kn + 32 * st + 8 * g4);
          rotate_row(src, nullptr, P->rope_new[jn][0], P->rope_new[jn][1], 1.0, row, nullptr);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rv = key0 + 4 * g4 + j;
        if (rv >= ke) continue;
        const int jn = new_index(rv);
        if (jn >= 0)
          VC::store(Vp + rv * rs + CW * c,
                    VC::template from_input<SF>(VC::load(a.vnew + new_off(jn) + CW * c)));
      }
    }
    load_tile(first, tb[0], lim0);
    load_tile(key_of(1), tb[1], lim0);
  }

  // Re-base tables for the in-loop rotation (float32, from the float64 plan).
  static_assert(D / 2 <= 64, "one rotary pair per lane of wave 0");
  if (KIND == kDecodeFused && delta != 0 && wave == 0 && lane < D / 2)
    sm_dt[lane] = rebase_table_entry(dt_c, dt_s);

  __syncthreads();  // the query operand (and the decoder's new row) is in LDS

  // encoder mask bookkeeping
  const int64_t last_pos = plan_t;
  const int slot_last = (slot_new + nnew - 1) % cap;
  const int64_t qpos = plan_pos + col_q;

  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x4 oacc[CW];
#pragma unroll
  for (int e = 0; e < CW; ++e) oacc[e] = f32x4{0.f, 0.f, 0.f, 0.f};

  // reb: std::integral_constant<bool, re-base this launch's tiles>
  auto process = [&](Tile& T, int key0, auto reb) __attribute__((always_inline)) {
    if (KL) {
      // fix_k: from the line layout to the operand layout (key key0 + c,
      // chunk 4 st + g4).  For line ln, operand st = 2 ln + s of lane m takes
      // the word of load 2 ln + (bit 3 of m) from lane m with bit 3 set to s:
      // the same lane, or its partner 8 lanes away (a row rotation by 8).
      const bool hi = (lane & 8) != 0;
#pragma unroll
      for (int ln = 0; ln < KS / 2; ++ln) {
        const u32x4 x0 = T.k[2 * ln], x1 = T.k[2 * ln + 1];
        u32x4 r0, r1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t a1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x1[e], 0x128, 0xF, 0xF, false);
          const uint32_t a0 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x0[e], 0x128, 0xF, 0xF, false);
          r0[e] = hi ? a1 : x0[e];
          r1[e] = hi ? x1[e] : a0;
        }
        T.k[2 * ln] = r0;
        T.k[2 * ln + 1] = r1;
      }
    }
    if (KIND == kDecodeFused && decltype(reb)::value && delta != 0) {
      __builtin_amdgcn_sched_barrier(0);
      // Exact re-base of the tile's rows in registers (R(-D), float32, rounded
      // to nearest bfloat16), written back for every valid row but the new
      // one, whose slot receives the appended row.
      const int row = key0 + c;
#pragma unroll
      for (int st = 0; st < KH; ++st) {
        const int i0 = 32 * st + 8 * g4;
        u32x4 dl = u32x4{0u, 0u, 0u, 0u}, dh = dl;
        rebase_chunks_ff<LO, SF>(T.k[st], T.k[st + KH], LO ? T.lo[st % (LO ? KS : 1)] : dl,
                             LO ? T.lo[(st + KH) % (LO ? KS : 1)] : dh,
                             [&](int e) { return sm_dt[i0 + e]; });
      }
      if (row < ke && row != slot_new) {
#pragma unroll
        for (int st = 0; st < KS; ++st) {
          st16(Kp + row * rs + 32 * st + 8 * g4, T.k[st]);
          if (LO) st16(Lp + row * rs + 32 * st + 8 * g4, T.lo[st % (LO ? KS : 1)]);
        }
      }
      // keep the re-base and the attention math apart (register pressure)
      __builtin_amdgcn_sched_barrier(0);
    }
    if (KIND == kDecodeFused && slot_new >= key0 && slot_new < key0 + TK) {
      // the new row lies in this tile: take its rotated K and V from LDS
      const int r = slot_new - key0;
      if (c == r) {
#pragma unroll
        for (int st = 0; st < KS; ++st) T.k[st] = sm_newk[st][g4];
      }
      if (g4 == (r >> 2)) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (j == (r & 3)) T.v[j] = sm_newv[c];
      }
    }
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < KS; ++st)
      acc = Mfma<SF>::scores(T.k[st], sm_q[st][lane], acc);
    float sv[4];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = (acc[r] + dpp_ror8(acc[r])) * a.scale_log2;
      const int row = key0 + 4 * g4 + r;
      bool vis = row < ke;
      if (KIND == kEncoderFused) {
        const int back = (slot_last - row + cap) % cap;
        const int64_t kpos = last_pos - back;
        vis = vis && kpos >= first_pos && kpos <= qpos;
      }
      x = vis ? x : -INFINITY;
      sv[r] = x;
      mx = fmaxf(mx, x);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool need = mx > m_run + kLazyMax;
    if (__any(need)) {
      const float alpha = need ? fast_exp2(m_run - mx) : 1.f;  // exp2(-inf) = 0
      if (need) m_run = mx;
      l_run *= alpha;
#pragma unroll
      for (int e = 0; e < CW; ++e) oacc[e] *= alpha;
    }
    float pj[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pj[r] = m_run == -INFINITY ? 0.f : fast_exp2(sv[r] - m_run);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool live = key0 + 4 * g4 + j < ke;
#pragma unroll
      for (int w = 0; w < CW / 2; ++w) T.v[j][w] = live ? T.v[j][w] : 0u;
    }
    l_run += (pj[0] + pj[1]) + (pj[2] + pj[3]);
    const uint32_t h01 = SF::cvt2(pj[0], pj[1]);
    const uint32_t h23 = SF::cvt2(pj[2], pj[3]);
    const uint32_t l01 = SF::cvt2(pj[0] - SF::to_f(h01 & 0xffffu), pj[1] - SF::to_f(h01 >> 16));
    const uint32_t l23 = SF::cvt2(pj[2] - SF::to_f(h23 & 0xffffu), pj[3] - SF::to_f(h23 >> 16));
    const uint32_t p01 = part ? l01 : h01;
    const uint32_t p23 = part ? l23 : h23;
    const u32x2 pop = u32x2{p01, p23};

    // V^T operand: dims CW*c + e of the tile's 4 keys of this lane group
#pragma unroll
    for (int e = 0; e < CW; ++e) {
      const int wd = e >> 1;
      const uint32_t w0 = (e & 1) ? pack_hi(T.v[0][wd], T.v[1][wd]) : pack_lo(T.v[0][wd], T.v[1][wd]);
      const uint32_t w1 = (e & 1) ? pack_hi(T.v[2][wd], T.v[3][wd]) : pack_lo(T.v[2][wd], T.v[3][wd]);
      oacc[e] = Mfma<SF>::pv(u32x2{w0, w1}, pop, oacc[e]);
    }
  };

  // ---- main loop: two tiles in registers, the one just used reloading ----
  // The trip count is uniform and the loads unconditional inside the loop, so
  // the compiler keeps the next tile's loads in flight across the current
  // tile's math (a conditional load makes it wait for every outstanding load).
  const int lim = lim0;
  auto run_tiles = [&](auto reb) __attribute__((always_inline)) {
    Tile& t0 = tb[0];
    Tile& t1 = tb[1];
    // tiles 0 and 1 are already in flight
    int i = 0;
    if (ntiles > 2) {
      process(t0, key_of(0), reb);
      load_tile(key_of(2), t0, lim);
      process(t1, key_of(1), reb);
      i = 2;
      for (; i + 2 < ntiles; i += 2) {
        load_tile(key_of(i + 1), t1, lim);
        process(t0, key_of(i), reb);
        load_tile(key_of(i + 2), t0, lim);
        process(t1, key_of(i + 1), reb);
      }
      if (ntiles - i == 2) {
        load_tile(key_of(i + 1), t1, lim);
        process(t0, key_of(i), reb);
        process(t1, key_of(i + 1), reb);
      } else {
        process(t0, key_of(i), reb);
      }
    } else if (ntiles == 2) {
      process(t0, key_of(0), reb);
      process(t1, key_of(1), reb);
    } else {
      process(t0, key_of(0), reb);
    }
  };
  if (ntiles > 0) run_tiles(std::integral_constant<bool, true>());

  // Delay conditioning of an unsplit item: the writing lanes request their
  // gamma and beta now, so the wave merge below hides the loads' latency.
  const int tc_hidden = a.Hkv * a.G * D;
  const bool tc_on = KIND != kEncoderFused && a.nsplit == 1 && tc_c >= 0 && tc_c < a.tc_conds;
  f32x4 tc_g[CW], tc_b[CW];
  if (tc_on && wave == 0 && c < 8 && c < a.G) {
    const float* tg = a.tc_mod + ((int64_t)l * a.tc_conds + tc_c) * 2 * tc_hidden +
                      (g * a.G + c) * D + 4 * CW * g4;
#pragma unroll
    for (int q4 = 0; q4 < CW; ++q4) {
      tc_g[q4] = *reinterpret_cast<const f32x4*>(tg + 4 * q4);
      tc_b[q4] = *reinterpret_cast<const f32x4*>(tg + tc_hidden + 4 * q4);
    }
  }

  // ---- per-wave reduction: row sums over lane groups, hi+lo columns ----
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
#pragma unroll
  for (int e = 0; e < CW; ++e)
#pragma unroll
    for (int r = 0; r < 4; ++r) oacc[e][r] += dpp_ror8(oacc[e][r]);

  // ---- merge the waves in wave 0 ----
  // When the item's key range is split and the splits merge in this launch,
  // every wave stays for the hand-over (the last split's waves all merge).
  const bool merge_here = a.nsplit > 1 && a.tickets != nullptr;
  if (NW > 1) {
    if (wave > 0 && c < 8) {
      if (g4 == 0) {
        sm_m[wave][c] = m_run;
        sm_l[wave][c] = l_run;
      }
#pragma unroll
      for (int e = 0; e < CW; ++e) sm_o[wave - 1][e][8 * g4 + c] = oacc[e];
    }
    __syncthreads();
    if (wave > 0 && !merge_here) return;
    if (wave == 0 && c < 8) {
      float M = m_run;
#pragma unroll
      for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_m[w][c]);
      const float f0 = (M == -INFINITY || m_run == -INFINITY) ? 0.f : fast_exp2(m_run - M);
      l_run *= f0;
#pragma unroll
      for (int e = 0; e < CW; ++e) oacc[e] *= f0;
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        const float mw = sm_m[w][c];
        const float fw = (M == -INFINITY || mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
        l_run += fw * sm_l[w][c];
#pragma unroll
        for (int e = 0; e < CW; ++e) oacc[e] += fw * sm_o[w - 1][e][8 * g4 + c];
      }
      m_run = M;
    }
  }

  // ---- output (or split partial): dims [4*CW*g4, 4*CW*g4 + 4*CW) of column c ----
  const int h = c;
  const bool writer = wave == 0 && c < 8 && h < a.G;
  float o[4 * CW];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int e = 0; e < CW; ++e) o[CW * r + e] = oacc[e][r];
  const int d0 = 4 * CW * g4;
  if (a.nsplit == 1) {
    if (!writer) return;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const int64_t off = vec_off(h) + d0;
    if (a.out_f32) {
      float* op = reinterpret_cast<float*>(a.out) + off;
#pragma unroll
      for (int q4 = 0; q4 < CW; ++q4) {
        f32x4 v =
            f32x4{o[4 * q4] * inv, o[4 * q4 + 1] * inv, o[4 * q4 + 2] * inv, o[4 * q4 + 3] * inv};
        if (tc_on) {
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = fmaf(v[k], 1.0f + tc_g[q4][k], tc_b[q4][k]);
        }
        *reinterpret_cast<f32x4*>(op + 4 * q4) = v;
      }
    } else {
      uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + off;
#pragma unroll
      for (int q8 = 0; q8 < CW / 2; ++q8) {
        u32x4 w;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          w[k] = cvt2_bf16(o[8 * q8 + 2 * k] * inv, o[8 * q8 + 2 * k + 1] * inv);
        if (tc_on) {
          // modulate the stored (rounded) value, as a separate pass would
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int i = 8 * q8 + 2 * k;   // dims i, i + 1 of the lane's 4 CW
            const float y0 = fmaf(bf2f(w[k] & 0xffffu), 1.0f + tc_g[i >> 2][i & 3],
                                  tc_b[i >> 2][i & 3]);
            const float y1 = fmaf(bf2f(w[k] >> 16), 1.0f + tc_g[(i + 1) >> 2][(i + 1) & 3],
                                  tc_b[(i + 1) >> 2][(i + 1) & 3]);
            w[k] = f2bf(y0) | (f2bf(y1) << 16);
          }
        }
        st16(op + 8 * q8, w);
      }
    }
    return;
  }
  // Split partial: maxima [0, 8), sums [8, 16), numerators [16 + h*D + dim).
  const int64_t pf = partial_floats(D);
  float* ib = a.ws + (int64_t)item * a.nsplit * pf;  // this item's partials
  if (!merge_here) {
    if (!writer) return;
    float* pp = ib + split * pf;
    if (g4 == 0) {
      pp[h] = m_run;
      pp[8 + h] = l_run;
    }
#pragma unroll
    for (int q4 = 0; q4 < CW; ++q4)
      *reinterpret_cast<f32x4*>(pp + 16 + h * D + d0 + 4 * q4) =
          f32x4{o[4 * q4], o[4 * q4 + 1], o[4 * q4 + 2], o[4 * q4 + 3]};
    return;
  }
  // In-launch merge: store the partial with device-scope stores, wait for
  // them to complete, then take a ticket; the split that takes the last one
  // finds every other split's partial complete in memory and merges them.
  __shared__ uint32_t sm_ticket;
  const __amdgpu_buffer_rsrc_t pb = dev_buffer(ib, (uint32_t)(a.nsplit * pf * 4));
  if (wave == 0) {
    if (writer) {
      const int pb0 = split * (int)pf;
      if (g4 == 0) {
        st_dev(pb, 4 * (pb0 + h), m_run);
        st_dev(pb, 4 * (pb0 + 8 + h), l_run);
      }
#pragma unroll
      for (int q4 = 0; q4 < CW; ++q4)
        st_dev4(pb, 4 * (pb0 + 16 + h * D + d0 + 4 * q4),
                f32x4{o[4 * q4], o[4 * q4 + 1], o[4 * q4 + 2], o[4 * q4 + 3]});
    }
    wait_stores();
    if (lane == 0)
      sm_ticket = __hip_atomic_fetch_add(a.tickets + item, 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (sm_ticket != (uint32_t)(a.nsplit - 1)) return;
  asm volatile("" ::: "memory");  // the partial loads stay behind the ticket
  const float* tg =
      KIND == kEncoderFused ? nullptr : tcond_row(a, l, s, a.Hkv * a.G * D);
  merge_partials<D, NW * 64>(pb, a, vec_off(0), KIND == kEncoderFused ? (int64_t)a.Hkv * D : D,
                             (int)threadIdx.x, tg ? tg + g * a.G * D : nullptr);
  if (threadIdx.x == 0)
    __hip_atomic_store(a.tickets + item, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge the split partials of one item: out = sum_j 2^(m_j - M) num_j / sum_j 2^(m_j - M) l_j.
// One thread per (column, dim) output.  The splits' maxima and sums of one
// item are staged through LDS once and each column's weights computed once,
// and a thread issues the loads of all its partial numerators together, so a
// merge costs about two memory round trips however many splits there are.
// The sums run over the splits in order, as a plain loop would.
constexpr int kCombineThreads = 1024;
constexpr int kMaxSplits = 64;

template <int D, int KIND>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(AttnArgs a) {
  __shared__ float sm_m[kMaxSplits][8];
  __shared__ float sm_l[kMaxSplits][8];
  __shared__ float sm_f[kMaxSplits][8];
  __shared__ float sm_den[8];
  const int item = blockIdx.x;
  const int g = item % a.Hkv;
  const int s = (item / a.Hkv) % a.S;
  const int l = item / (a.Hkv * a.S);
  const int ns = a.nsplit;
  const int64_t pf = partial_floats(D);
  const float* base = a.ws + (int64_t)item * ns * pf;
  // A thread's partials of the first 8 splits are read at once, together with
  // the maxima and sums (they do not depend on them): one round trip to
  // memory for up to 8 splits instead of two.
  const int idx = threadIdx.x;
  const bool live = idx < a.G * D;
  const int h = live ? idx / D : 0;
  const int d = idx - h * D;
  const float* num_p = base + 16 + h * D + d;
  float v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) v[u] = live && u < ns ? num_p[u * pf] : 0.f;
  for (int i = threadIdx.x; i < ns * 8; i += kCombineThreads) {
    const int j = i >> 3, h = i & 7;
    sm_m[j][h] = base[j * pf + h];
    sm_l[j][h] = base[j * pf + 8 + h];
  }
  __syncthreads();
  if ((int)threadIdx.x < a.G) {
    const int hh = threadIdx.x;
    float M = -INFINITY;
    for (int j = 0; j < ns; ++j) M = fmaxf(M, sm_m[j][hh]);
    float den = 0.f;
    for (int j = 0; j < ns; ++j) {
      const float mj = sm_m[j][hh];
      const float f = (M == -INFINITY || mj == -INFINITY) ? 0.f : fast_exp2(mj - M);
      sm_f[j][hh] = f;
      den += f * sm_l[j][hh];
    }
    sm_den[hh] = den;
  }
  __syncthreads();
  if (!live) return;
  float num = 0.f;
  for (int j0 = 0; j0 < ns; j0 += 8) {
    if (j0 > 0) {
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = j0 + u < ns ? num_p[(j0 + u) * pf] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (j0 + u < ns) num += sm_f[j0 + u][h] * v[u];
  }
  const float den = sm_den[h];
  float o = den > 0.f ? num / den : 0.f;
  int64_t off;
  if (KIND == kEncoderFused) off = ((((int64_t)l * a.S + s) * a.F + h) * a.Hkv + g) * D + d;
  else off = ((((int64_t)l * a.S + s) * a.Hkv + g) * a.G + h) * D + d;
  if (KIND != kEncoderFused) {
    // delay conditioning of the stored value
    const int hidden = a.Hkv * a.G * D;
    const float* tg = tcond_row(a, l, s, hidden);
    if (tg) {
      const int i = (g * a.G + h) * D + d;
      const float x = a.out_f32 ? o : bf2f(f2bf(o));
      o = fmaf(x, 1.0f + tg[i], tg[hidden + i]);
    }
  }
  if (a.out_f32) reinterpret_cast<float*>(a.out)[off] = o;
  else reinterpret_cast<uint16_t*>(a.out)[off] = (uint16_t)f2bf(o);
}

// Waves per workgroup (one item each): 4, or 2 at d = 64 when a launch has
// many items.  Then an item's rows are half as long and the shorter-lived,
// more numerous workgroups keep the memory queue fuller: the 32-layer
// encoder launch (81,920 items) runs 5 % faster with 2 (3 and 6 were
// slower); a one-layer encoder launch (2,560 items, under 2 rounds of
// resident 2-wave workgroups) is faster with 4, as is every d = 128 case.
constexpr int64_t kManyItems = 12288;

template <int D, int NW, int KIND, bool COMP, typename SF, bool KL>
hipError_t launch_nw(const AttnArgs& args, int items, hipStream_t stream) {
  const int extra = args.adv_state ? (args.S + NW - 1) / NW
                                    : (KIND == kEncoderFused && args.pull ? args.pull_blocks : 0);
  hipLaunchKernelGGL((attn_kernel<D, NW, KIND, COMP, SF, KL>),
                     dim3(items * args.nsplit + extra), dim3(NW * 64), 0, stream, args);
  return hipGetLastError();
}

// Decoder launches whose workgroups stream at most this many rows read K as
// whole lines with the non-temporal hint (the key-tile loads in the operand
// layout touch half lines, which the hint makes slower).  Measured on the
// same launches, same bits: 36 x 64 at W = 375 (375 rows) 157.4 -> 153.6 us,
// 36 x 256 mixed windows pipelined 507 -> 497 us, 26 x 16 compaction at
// W = 8192 split 24 ways (342 rows) 697 -> 682 us; but split 8 ways (1,024
// rows) 581 -> 588 us and 3 ways (2,736 rows) 558 -> 568 us, and the d = 64
// encoder chunks (754 rows) 2.64 -> 2.67 ms.
constexpr int kLineRows = 512;

template <int D, int KIND, bool COMP, typename SF>
hipError_t launch_kind(const AttnArgs& args, int items, hipStream_t stream) {
  hipError_t e;
  const int per = (((args.ring.slots + args.nsplit - 1) / args.nsplit) + 15) & ~15;
  if constexpr (D == 128 && KIND != kEncoderFused) {
    if (per <= kLineRows)
      e = launch_nw<D, 4, KIND, COMP, SF, true>(args, items, stream);
    else
      e = launch_nw<D, 4, KIND, COMP, SF, false>(args, items, stream);
  } else {
    if (D == 64 && (int64_t)items * args.nsplit >= kManyItems)
      e = launch_nw<D, 2, KIND, COMP, SF, false>(args, items, stream);
    else
      e = launch_nw<D, 4, KIND, COMP, SF, false>(args, items, stream);
  }
  if (e != hipSuccess || args.nsplit == 1 || args.tickets) return e;
  hipLaunchKernelGGL((combine_kernel<D, KIND>), dim3(items), dim3(kCombineThreads), 0, stream,
                     args);
  return hipGetLastError();
}

template <int D, typename SF>
hipError_t launch_dec(AttnKind kind, bool comp, const AttnArgs& args, int items,
                      hipStream_t stream) {
  if (kind == kDecodeRead) return launch_kind<D, kDecodeRead, false, SF>(args, items, stream);
  return comp ? launch_kind<D, kDecodeFused, true, SF>(args, items, stream)
              : launch_kind<D, kDecodeFused, false, SF>(args, items, stream);
}

template <int D>
hipError_t launch_d(AttnKind kind, bool comp, bool f16, const AttnArgs& args, int items,
                    hipStream_t stream) {
  // the encoder stores bfloat16 only (the configuration check rejects fp16)
  if (kind == kEncoderFused)
    return launch_kind<D, kEncoderFused, false, StoreBf16>(args, items, stream);
  return f16 ? launch_dec<D, StoreF16>(kind, comp, args, items, stream)
             : launch_dec<D, StoreBf16>(kind, comp, args, items, stream);
}

}  // namespace

int choose_splits(const rkv_cfg* cfg, int32_t slots) {
  if (cfg->num_splits > 0) {
    int max_split = (slots + 15) / 16;
    if (max_split > kMaxSplits) max_split = kMaxSplits;
    return cfg->num_splits < max_split ? cfg->num_splits : (max_split > 0 ? max_split : 1);
  }
  // Enough workgroups to spread a small launch over the chip (about 2048),
  // but no split shorter than 256 keys: a short split's fixed costs and the
  // merge launch cost more than its parallelism gains (measured: one split
  // is fastest at W = 375 for any item count, six help at W = 2048 up to 32
  // items).  Re-basing every position with the residual costs several times
  // more per key, so there splits of about 48 keys still pay (measured at
  // W = 375, one item per head: 8 splits 12.8 us a step, 5 splits 14.1, 12
  // splits 13.4).
  const int64_t items = (int64_t)cfg->num_layers * cfg->num_streams * cfg->num_kv_heads;
  const int64_t target = 2048;
  int64_t n = (target + items - 1) / items;
  const bool heavy = (cfg->flags & RKV_F_COMPENSATED) && cfg->rebase_chunk == 1;
  const int64_t max_split = heavy ? (slots + 24) / 48 : slots / 256;
  if (n > max_split) n = max_split;
  if (n > kMaxSplits) n = kMaxSplits;
  if (n < 1) n = 1;
  return (int)n;
}

hipError_t launch_attention(const rkv_cfg* cfg, AttnKind kind, const AttnArgs& args,
                            hipStream_t stream) {
  const int items = cfg->num_layers * cfg->num_streams * cfg->num_kv_heads;
  const bool comp = (cfg->flags & RKV_F_COMPENSATED) != 0;
  const bool f16 = (cfg->flags & RKV_F_KV_FP16) != 0;
  if (cfg->head_dim == 128) return launch_d<128>(kind, comp, f16, args, items, stream);
  return launch_d<64>(kind, comp, f16, args, items, stream);
}

}  // namespace rkv
