// Incremental encoder step through a stack of layers (voxtral.c explainer,
// section 三: the causal encoder computes only the new positions of a step,
// each layer attending from them to its cached K/V; Audio8 explainer's
// table: 32 layers, hidden 1280, a 750-frame window).  Each layer is
//
//   a = RMSNorm(x) g1;  q, k, v = a Wq^T, a Wk^T, a Wv^T
//   x += Wo attn(q, k, v)                       (rkv_encoder_chunk_attn)
//   x += W2 gelu(W1 RMSNorm(x) g2)
//
// with the residual stream x in float32 and every other activation in
// bfloat16.  The projections are plain GEMMs on the matrix cores
// (v_mfma_f32_16x16x32_bf16, float32 accumulation): the weight matrix (row =
// output feature, contiguous in k) is the A operand and the activations (row
// = token) the B operand, so a lane's result holds four consecutive output
// features of one token and the epilogue writes them as one vector.  A
// workgroup computes 64 tokens x 64 features; each of its 4 waves a 32 x 32
// quarter, so every element read from LDS feeds 64 products instead of 16.
// With 512 tokens the products are short in M, and what bounds them is
// moving operands into and out of LDS, not the matrix cores: with both
// switched off, the q/k/v launch's loop of LDS writes, reads and barriers
// alone took 11.2 of its 13.1 us.  So the operand tiles go from global memory
// straight into LDS (gfx950's global_load_lds_dwordx4: no staging registers
// and no LDS write instructions) through a ring of NS k-stages, NS - 1 of them
// in flight.  With the weights cache-resident this takes q/k/v from 13.1 to
// 9.9 us and the up-projection from 16.2 to 12.3 us (same bits); in the
// encoder step each layer's weights come cold from HBM once, and there the
// first touch of the weight panels bounds the products (q/k/v 14.6 -> 14.3
// us).  Larger tiles (64 x 128, 128 x 64 per workgroup), weights loaded
// straight into the MFMA operand registers, and a block order that keeps a
// weight panel's token tiles on one XCD were slower.

#include <math.h>

#include "rkv_device.h"
#include "rkv_encoder.h"
#include "rkv_internal.h"

namespace rkv {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

enum Epilogue { kStoreBf16 = 0, kAddF32 = 1, kGeluBf16 = 2, kStoreF32 = 3 };

// Up to four GEMMs launched together: the q, k, v projections (one shared B
// operand), or the k-slices of one split product.
struct GemmSet {
  const uint16_t* w[kGemmMaxSet];   // [N][ld] bfloat16, k from 0 to K
  const uint16_t* x[kGemmMaxSet];   // [M][ld] bfloat16, k from 0 to K
  void* c[kGemmMaxSet];             // [M][N]: bfloat16, or float32 (kAddF32, kStoreF32)
};

__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

constexpr int kTM = 64, kTN = 64, kKS = 64;
// LDS tiles: rows of kKS elements (128 bytes) without padding; the eight
// 16-byte chunks of row r are stored in the order chunk ^ ((r >> 1) & 7).
// A 16-lane group of a 16-byte operand read takes one chunk of 16
// consecutive rows, which the swizzle puts on 16 distinct 4-bank groups of
// the 64 banks (rows padded to 144 bytes instead left the stores 2-way
// conflicted).
__device__ __forceinline__ int lds_at(int row, int chunk) {
  return row * kKS + 8 * (chunk ^ ((row >> 1) & 7));
}
// Wait until at most N of this wave's vector memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_loads() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
constexpr int kWF = kTN / 2;       // features per wave (2 x 2 waves: 32 tokens x 32 features)
constexpr int kFB = kWF / 16;      // 16-feature MFMA blocks per wave

template <int EP, int NS>
__global__ __launch_bounds__(256) void gemm_kernel(GemmSet set, int M, int N, int K, int ld) {
  static_assert(NS >= 2 && NS <= 3, "ring depth");
  // one k-stage: weight tile [64][kKS], then token tile [64][kKS]; a ring of
  // NS stages in separate arrays, so the compiler sees that a stage's reads
  // do not touch the stages still being loaded
  __shared__ __attribute__((aligned(16))) uint16_t st0[2 * 64 * kKS];
  __shared__ __attribute__((aligned(16))) uint16_t st1[2 * 64 * kKS];
  __shared__ __attribute__((aligned(16))) uint16_t st2[NS > 2 ? 2 * 64 * kKS : 8];
  auto stage = [&](int slot) -> uint16_t* { return slot == 0 ? st0 : slot == 1 ? st1 : st2; };
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;          // token half, feature half
  const int bz = blockIdx.z;
  const uint16_t* __restrict__ w = set.w[bz];
  const uint16_t* __restrict__ x = set.x[bz];
  const int n0 = blockIdx.x * kTN, m0 = blockIdx.y * kTM;
  // Loads: wave v moves rows [16 v, 16 v + 16) of both tiles, 8 rows (1 KB)
  // per instruction; lane i takes row r0 + i / 8 and lands in its chunk slot
  // i % 8, which holds logical chunk (i % 8) ^ ((row >> 1) & 7).  Token rows
  // past M and feature rows past N (N is a multiple of 64, so a last tile may
  // hold 64 features) are clamped: read, never stored.
  const uint16_t* src[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 16 * wave + 8 * h + (lane >> 3);
    const int q = (lane & 7) ^ ((row >> 1) & 7);
    src[0][h] = w + (int64_t)min(n0 + row, N - 1) * ld + 8 * q;
    src[1][h] = x + (int64_t)min(m0 + row, M - 1) * ld + 8 * q;
  }
  const int steps = K / kKS;
  auto issue = [&](int s, int slot) __attribute__((always_inline)) {
    const int k0 = (s < steps ? s : steps - 1) * kKS;   // past the end: a harmless reload
#pragma unroll
    for (int o = 0; o < 2; ++o)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        lds_dma16(src[o][h] + k0, stage(slot) + (o * 64 + 16 * wave + 8 * h) * kKS);
  };
  f32x4 acc[2][kFB];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < kFB; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto frag = [&](int slot, int kk, bf16x8* fa, bf16x8* fb) __attribute__((always_inline)) {
    const uint16_t* b = stage(slot);
#pragma unroll
    for (int i = 0; i < kFB; ++i)
      fa[i] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(&b[lds_at(wn * kWF + 16 * i + c, (kk >> 3) + g)]));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      fb[j] = __builtin_bit_cast(
          bf16x8,
          *reinterpret_cast<const u32x4*>(&b[lds_at(64 + wm * 32 + 16 * j + c, (kk >> 3) + g)]));
  };
  auto mma = [&](const bf16x8* fa, const bf16x8* fb) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < kFB; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[j][i], 0, 0, 0);
  };
  static_assert(kKS == 64, "a k-stage is two 32-k chunks");
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s, s);
  bf16x8 fa0[kFB], fb0[2], fa1[kFB], fb1[2];
  for (int s0 = 0; s0 < steps; s0 += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int s = s0 + u;
      if (s < steps) {
        // this wave's 4 loads of stage s are in LDS (those of the NS - 2
        // later stages may still be in flight) ...
        wait_loads<4 * (NS - 2)>();
        // ... and every wave's are; every wave has also finished reading
        // stage s - 1, whose slot is loaded next
        __builtin_amdgcn_s_barrier();
        issue(s + NS - 1, (u + NS - 1) % NS);
        frag(u, 0, fa0, fb0);
        frag(u, 32, fa1, fb1);
        mma(fa0, fb0);
        mma(fa1, fb1);
      }
    }
  }
  // lane (c, g) of acc[j][i] holds features n0 + kWF wn + 16 i + 4 g + r, r < 4,
  // of token m0 + 32 wm + 16 j + c
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = m0 + 32 * wm + 16 * j + c;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < kFB; ++i) {
      const f32x4 v = acc[j][i];
      const int n = n0 + kWF * wn + 16 * i + 4 * g;
      if (n >= N) continue;
      if (EP == kAddF32) {
        float* p = reinterpret_cast<float*>(set.c[bz]) + (int64_t)m * N + n;
        const f32x4 old = *reinterpret_cast<const f32x4*>(p);
        *reinterpret_cast<f32x4*>(p) = old + v;
      } else if (EP == kStoreF32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(set.c[bz]) + (int64_t)m * N +
                                  n) = v;
      } else {
        float e0 = v[0], e1 = v[1], e2 = v[2], e3 = v[3];
        if (EP == kGeluBf16) {
          e0 = gelu_erf(e0);
          e1 = gelu_erf(e1);
          e2 = gelu_erf(e2);
          e3 = gelu_erf(e3);
        }
        uint16_t* p = reinterpret_cast<uint16_t*>(set.c[bz]) + (int64_t)m * N + n;
        *reinterpret_cast<u32x2*>(p) = u32x2{cvt2_bf16(e0, e1), cvt2_bf16(e2, e3)};
      }
    }
  }
}

// x[m] += part_0[m] + ... + part_{NP-1}[m] (in that order), then
// a[m] = bf16(x[m] / sqrt(mean(x[m]^2) + eps) * g) unless a is null: one
// workgroup per token row, each thread up to kNormPerThread float4 of it,
// held in registers throughout; every load of the row is issued at once.
template <int NP>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(
    float* __restrict__ x, const float* __restrict__ parts, int64_t part_stride,
    const uint16_t* __restrict__ g, uint16_t* __restrict__ a, int hidden, float eps) {
  __shared__ float red[kNormThreads / 64];
  const int t = threadIdx.x;
  const int n4 = hidden >> 2;
  const int64_t row = (int64_t)blockIdx.x * hidden;
  f32x4* xr = reinterpret_cast<f32x4*>(x + row);
  const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 v[kNormPerThread], pv[NP > 0 ? NP : 1][kNormPerThread];
#pragma unroll
  for (int j = 0; j < kNormPerThread; ++j) {
    const int i = t + kNormThreads * j;
    v[j] = i < n4 ? xr[i] : zero;
#pragma unroll
    for (int p = 0; p < NP; ++p)
      pv[p][j] = i < n4 ? reinterpret_cast<const f32x4*>(parts + p * part_stride + row)[i] : zero;
  }
  if (NP > 0) {
#pragma unroll
    for (int j = 0; j < kNormPerThread; ++j) {
#pragma unroll
      for (int p = 0; p < NP; ++p) v[j] += pv[p][j];
      const int i = t + kNormThreads * j;
      if (i < n4) xr[i] = v[j];
    }
  }
  if (!a) return;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kNormPerThread; ++j)
    ss = fmaf(v[j][0], v[j][0], fmaf(v[j][1], v[j][1], fmaf(v[j][2], v[j][2],
                                                             fmaf(v[j][3], v[j][3], ss))));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if ((t & 63) == 0) red[t >> 6] = ss;
  __syncthreads();
  ss = 0.f;
#pragma unroll
  for (int w = 0; w < kNormThreads / 64; ++w) ss += red[w];
  const float r = 1.0f / sqrtf(ss / (float)hidden + eps);
  uint16_t* ar = a + row;
#pragma unroll
  for (int j = 0; j < kNormPerThread; ++j) {
    const int i = t + kNormThreads * j;
    if (i < n4) {
      const u32x2 gg = *reinterpret_cast<const u32x2*>(g + 4 * i);
      *reinterpret_cast<u32x2*>(ar + 4 * i) =
          u32x2{cvt2_bf16(v[j][0] * r * bf2f(gg[0] & 0xffffu), v[j][1] * r * bf2f(gg[0] >> 16)),
                cvt2_bf16(v[j][2] * r * bf2f(gg[1] & 0xffffu), v[j][3] * r * bf2f(gg[1] >> 16))};
    }
  }
}

}  // namespace

hipError_t launch_rmsnorm(float* x, const float* parts, int nparts, int64_t part_stride,
                          const uint16_t* g, uint16_t* a, int M, int hidden, float eps,
                          hipStream_t stream) {
  const dim3 grid(M), block(kNormThreads);
  switch (nparts) {
    case 0:
      hipLaunchKernelGGL(rmsnorm_kernel<0>, grid, block, 0, stream, x, parts, part_stride, g, a,
                         hidden, eps);
      break;
    case 1:
      hipLaunchKernelGGL(rmsnorm_kernel<1>, grid, block, 0, stream, x, parts, part_stride, g, a,
                         hidden, eps);
      break;
    case 2:
      hipLaunchKernelGGL(rmsnorm_kernel<2>, grid, block, 0, stream, x, parts, part_stride, g, a,
                         hidden, eps);
      break;
    case 4:
      hipLaunchKernelGGL(rmsnorm_kernel<4>, grid, block, 0, stream, x, parts, part_stride, g, a,
                         hidden, eps);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(GemmEpilogue ep, const uint16_t* const* w, const uint16_t* const* x,
                       void* const* c, int count, int M, int N, int K, int ld,
                       hipStream_t stream) {
  GemmSet set{};
  for (int i = 0; i < count; ++i) {
    set.w[i] = w[i];
    set.x[i] = x[i];
    set.c[i] = c[i];
  }
  const dim3 grid((N + kTN - 1) / kTN, (M + kTM - 1) / kTM, count);
  // Three k-stages in the ring (two in flight), or two for short products
  // (fewer than 10 k-stages), whose prologue the deeper ring does not repay.
  // Measured at 512 tokens with each product's weights read cold from HBM,
  // as in the encoder step, old kernel -> two -> three stages: q/k/v 14.6 ->
  // 17.3 -> 14.3 us, up-projection 18.8 -> 19.7 -> 18.2, down-projection
  // 18.4 -> 19.4 -> 18.4, output projection (k-slices of 320) 7.8 -> 7.0 ->
  // 7.4; with the weights cache-resident q/k/v takes 13.0 -> 11.2 -> 9.9 us.
  const bool deep = K / kKS >= 10;
  switch (ep) {
    case GemmEpilogue::kStoreBf16:
      if (deep)
        hipLaunchKernelGGL((gemm_kernel<kStoreBf16, 3>), grid, dim3(256), 0, stream, set, M, N, K, ld);
      else
        hipLaunchKernelGGL((gemm_kernel<kStoreBf16, 2>), grid, dim3(256), 0, stream, set, M, N, K, ld);
      break;
    case GemmEpilogue::kAddF32:
      hipLaunchKernelGGL((gemm_kernel<kAddF32, 2>), grid, dim3(256), 0, stream, set, M, N, K, ld);
      break;
    case GemmEpilogue::kGeluBf16:
      if (deep)
        hipLaunchKernelGGL((gemm_kernel<kGeluBf16, 3>), grid, dim3(256), 0, stream, set, M, N, K, ld);
      else
        hipLaunchKernelGGL((gemm_kernel<kGeluBf16, 2>), grid, dim3(256), 0, stream, set, M, N, K, ld);
      break;
    default:
      if (deep)
        hipLaunchKernelGGL((gemm_kernel<kStoreF32, 3>), grid, dim3(256), 0, stream, set, M, N, K, ld);
      else
        hipLaunchKernelGGL((gemm_kernel<kStoreF32, 2>), grid, dim3(256), 0, stream, set, M, N, K, ld);
      break;
  }
  return hipGetLastError();
}

}  // namespace rkv
