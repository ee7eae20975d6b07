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
// workgroup computes 64 tokens x 64 features: both operand tiles of a
// k-stage are staged through LDS (double-buffered; the global loads of the
// next kDepth stages are in flight during a stage's MFMAs), and each of the 4
// waves computes a 32 x 32 quarter from them, so every loaded element feeds
// 64 products instead of 16.  Two workgroups share a CU (two waves per
// SIMD): a 64 x 128 tile (one workgroup per CU at 512 tokens, 0.75 instead of
// one operand read per product) measured slower, its single wave per SIMD
// left with nothing to run while it waits for LDS.

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
// consecutive rows and a group of a staging write two whole rows: either
// way the swizzle puts the 16 pieces on 16 distinct 4-bank groups of the 64
// banks.  (Rows padded to 144 bytes left the staging writes 2-way conflicted:
// the bank-conflict counter read as many cycles as LDS instructions were
// active.)
__device__ __forceinline__ int lds_at(int row, int chunk) {
  return row * kKS + 8 * (chunk ^ ((row >> 1) & 7));
}
constexpr int kDepth = 2;          // k-stages whose global loads are in flight
constexpr int kWF = kTN / 2;       // features per wave (2 x 2 waves: 32 tokens x 32 features)
constexpr int kFB = kWF / 16;      // 16-feature MFMA blocks per wave
constexpr int kWRows = kTN / 32;   // weight rows each thread stages per k-stage

template <int EP>
__global__ __launch_bounds__(256) void gemm_kernel(GemmSet set, int M, int N, int K, int ld) {
  __shared__ __attribute__((aligned(16))) uint16_t sw[2][kTN * kKS];
  __shared__ __attribute__((aligned(16))) uint16_t sx[2][kTM * kKS];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;          // token half, feature half
  const uint16_t* __restrict__ w = set.w[blockIdx.z];
  const uint16_t* __restrict__ x = set.x[blockIdx.z];
  const int n0 = blockIdx.x * kTN, m0 = blockIdx.y * kTM;
  // staging: thread t moves the 16-byte pieces (row t/8 + 32 r, k 8 (t%8)) of
  // both tiles; token rows past M and feature rows past N (N is a multiple of
  // 64, so a last tile may hold 64 features) are clamped: read, never stored
  const int lr = t >> 3, lk = 8 * (t & 7);
  const uint16_t* wp[kWRows];
#pragma unroll
  for (int r = 0; r < kWRows; ++r) wp[r] = w + (int64_t)min(n0 + 32 * r + lr, N - 1) * ld + lk;
  const uint16_t* xp0 = x + (int64_t)min(m0 + lr, M - 1) * ld + lk;
  const uint16_t* xp1 = x + (int64_t)min(m0 + 32 + lr, M - 1) * ld + lk;
  const int steps = K / kKS;
  // register ring: stage s's pieces sit in slot s % kDepth from its load until
  // its LDS store, which frees the slot for stage s + kDepth
  u32x4 rw[kDepth][kWRows], rx0[kDepth], rx1[kDepth];
  auto gload = [&](int s, int slot) {
    const int k0 = (s < steps ? s : steps - 1) * kKS;   // past the end: a harmless reload
#pragma unroll
    for (int r = 0; r < kWRows; ++r) rw[slot][r] = ld16(wp[r] + k0);
    rx0[slot] = ld16(xp0 + k0);
    rx1[slot] = ld16(xp1 + k0);
  };
  auto lstore = [&](int b, int slot) {
    const int ch = lk >> 3;
#pragma unroll
    for (int r = 0; r < kWRows; ++r)
      *reinterpret_cast<u32x4*>(&sw[b][lds_at(32 * r + lr, ch)]) = rw[slot][r];
    *reinterpret_cast<u32x4*>(&sx[b][lds_at(lr, ch)]) = rx0[slot];
    *reinterpret_cast<u32x4*>(&sx[b][lds_at(32 + lr, ch)]) = rx1[slot];
  };
  f32x4 acc[2][kFB];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < kFB; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // operand fragments of one 32-k chunk: the next chunk's are read from LDS
  // before this chunk's products are issued, so the LDS latency hides behind
  // them (read and used at once, the wave waits for every read)
  auto frag = [&](int b, int kk, bf16x8* fa, bf16x8* fb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kFB; ++i)
      fa[i] = __builtin_bit_cast(
          bf16x8,
          *reinterpret_cast<const u32x4*>(&sw[b][lds_at(wn * kWF + 16 * i + c, (kk >> 3) + g)]));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      fb[j] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(&sx[b][lds_at(wm * 32 + 16 * j + c, (kk >> 3) + g)]));
  };
  auto mma = [&](const bf16x8* fa, const bf16x8* fb) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < kFB; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[j][i], 0, 0, 0);
  };
  static_assert(kKS == 64, "a k-stage is two 32-k chunks");
  bf16x8 fa0[kFB], fb0[2], fa1[kFB], fb1[2];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) gload(d, d);
  lstore(0, 0);
  gload(kDepth, 0);
  __syncthreads();
  frag(0, 0, fa0, fb0);
  for (int s0 = 0; s0 < steps; s0 += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      const int s = s0 + u;
      if (s < steps) {
        const int b = u & 1;                            // kDepth even: s & 1
        frag(b, 32, fa1, fb1);
        mma(fa0, fb0);
        // the LDS buffer written here was last read in stage s - 1, which every
        // wave finished before the barrier that ended it
        if (s + 1 < steps) {
          const int slot = (u + 1) % kDepth;
          lstore(b ^ 1, slot);
          if (s + 1 + kDepth < steps) gload(s + 1 + kDepth, slot);
        }
        mma(fa1, fb1);
        __syncthreads();
        if (s + 1 < steps) frag(b ^ 1, 0, fa0, fb0);
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
        float* p = reinterpret_cast<float*>(set.c[blockIdx.z]) + (int64_t)m * N + n;
        const f32x4 old = *reinterpret_cast<const f32x4*>(p);
        *reinterpret_cast<f32x4*>(p) = old + v;
      } else if (EP == kStoreF32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(set.c[blockIdx.z]) + (int64_t)m * N +
                                  n) = v;
      } else {
        float e0 = v[0], e1 = v[1], e2 = v[2], e3 = v[3];
        if (EP == kGeluBf16) {
          e0 = gelu_erf(e0);
          e1 = gelu_erf(e1);
          e2 = gelu_erf(e2);
          e3 = gelu_erf(e3);
        }
        uint16_t* p = reinterpret_cast<uint16_t*>(set.c[blockIdx.z]) + (int64_t)m * N + n;
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
  switch (ep) {
    case GemmEpilogue::kStoreBf16:
      hipLaunchKernelGGL((gemm_kernel<kStoreBf16>), grid, dim3(256), 0, stream, set, M, N, K, ld);
      break;
    case GemmEpilogue::kAddF32:
      hipLaunchKernelGGL((gemm_kernel<kAddF32>), grid, dim3(256), 0, stream, set, M, N, K, ld);
      break;
    case GemmEpilogue::kGeluBf16:
      hipLaunchKernelGGL((gemm_kernel<kGeluBf16>), grid, dim3(256), 0, stream, set, M, N, K, ld);
      break;
    default:
      hipLaunchKernelGGL((gemm_kernel<kStoreF32>), grid, dim3(256), 0, stream, set, M, N, K, ld);
      break;
  }
  return hipGetLastError();
}

}  // namespace rkv
