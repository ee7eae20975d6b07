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
// workgroup of 4 waves computes 64 tokens x 32 features, each wave 16 tokens;
// the operands of the next two k-steps are in flight while one is computed.

#include <math.h>

#include "rkv_device.h"
#include "rkv_encoder.h"
#include "rkv_internal.h"

namespace rkv {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

enum Epilogue { kStoreBf16 = 0, kAddF32 = 1, kGeluBf16 = 2 };

// Up to three GEMMs sharing the B operand (the q, k, v projections).
struct GemmSet {
  const uint16_t* w[3];   // [N][K] bfloat16
  void* c[3];             // [M][N]: bfloat16, or float32 (kAddF32)
};

__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

template <int EP>
__global__ __launch_bounds__(256) void gemm_kernel(GemmSet set, const uint16_t* __restrict__ x,
                                                   int M, int N, int K) {
  constexpr int TM = 64, TN = 32, KS = 32;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g4 = lane >> 4;
  const uint16_t* __restrict__ w = set.w[blockIdx.z];
  const int n0 = blockIdx.x * TN;
  const int m0 = blockIdx.y * TM + 16 * wave;
  const int mrow = m0 + c < M ? m0 + c : M - 1;          // ragged M: clamp, not stored
  const uint16_t* xr = x + (int64_t)mrow * K + 8 * g4;
  const uint16_t* w0 = w + (int64_t)(n0 + c) * K + 8 * g4;
  const uint16_t* w1 = w + (int64_t)(n0 + 16 + c) * K + 8 * g4;
  f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  const int steps = K / KS;
  u32x4 bx[3], aw0[3], aw1[3];
  auto load = [&](int i, int slot) {
    const int k0 = (i < steps ? i : steps - 1) * KS;
    bx[slot] = ld16(xr + k0);
    aw0[slot] = ld16(w0 + k0);
    aw1[slot] = ld16(w1 + k0);
  };
  load(0, 0);
  load(1, 1);
  for (int i = 0; i < steps; i += 3) {
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      if (i + u < steps) {
        load(i + u + 2, (u + 2) % 3);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, aw0[u]),
                                                       __builtin_bit_cast(bf16x8, bx[u]), acc0,
                                                       0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, aw1[u]),
                                                       __builtin_bit_cast(bf16x8, bx[u]), acc1,
                                                       0, 0, 0);
      }
    }
  }
  // lane (c, g4) holds features n0 + 4 g4 + r (acc0) and n0 + 16 + 4 g4 + r
  // (acc1), r < 4, of token m0 + c
  const int m = m0 + c;
  if (m >= M) return;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const f32x4 v = h ? acc1 : acc0;
    const int n = n0 + 16 * h + 4 * g4;
    if (EP == kAddF32) {
      float* p = reinterpret_cast<float*>(set.c[blockIdx.z]) + (int64_t)m * N + n;
      f32x4 old = *reinterpret_cast<const f32x4*>(p);
      *reinterpret_cast<f32x4*>(p) = old + v;
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

// a[m] = bf16(x[m] / sqrt(mean(x[m]^2) + eps) * g): one wave per token row.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x,
                                                      const uint16_t* __restrict__ g,
                                                      uint16_t* __restrict__ a, int M, int hidden,
                                                      float eps) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  const float* xr = x + (int64_t)m * hidden;
  float ss = 0.f;
  for (int i = 2 * lane; i < hidden; i += 128) {
    const f32x2 v = *reinterpret_cast<const f32x2*>(xr + i);
    ss = fmaf(v[0], v[0], fmaf(v[1], v[1], ss));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  const float r = 1.0f / sqrtf(ss / (float)hidden + eps);
  uint16_t* ar = a + (int64_t)m * hidden;
  for (int i = 2 * lane; i < hidden; i += 128) {
    const f32x2 v = *reinterpret_cast<const f32x2*>(xr + i);
    const uint32_t gg = *reinterpret_cast<const uint32_t*>(g + i);
    *reinterpret_cast<uint32_t*>(ar + i) =
        cvt2_bf16(v[0] * r * bf2f(gg & 0xffffu), v[1] * r * bf2f(gg >> 16));
  }
}

}  // namespace

hipError_t launch_rmsnorm(const float* x, const uint16_t* g, uint16_t* a, int M, int hidden,
                          float eps, hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((M + 3) / 4), dim3(256), 0, stream, x, g, a, M, hidden,
                     eps);
  return hipGetLastError();
}

hipError_t launch_gemm(GemmEpilogue ep, const uint16_t* const* w, void* const* c, int count,
                       const uint16_t* x, int M, int N, int K, hipStream_t stream) {
  GemmSet set{};
  for (int i = 0; i < count; ++i) {
    set.w[i] = w[i];
    set.c[i] = c[i];
  }
  const dim3 grid(N / 32, (M + 63) / 64, count);
  switch (ep) {
    case GemmEpilogue::kStoreBf16:
      hipLaunchKernelGGL((gemm_kernel<kStoreBf16>), grid, dim3(256), 0, stream, set, x, M, N, K);
      break;
    case GemmEpilogue::kAddF32:
      hipLaunchKernelGGL((gemm_kernel<kAddF32>), grid, dim3(256), 0, stream, set, x, M, N, K);
      break;
    default:
      hipLaunchKernelGGL((gemm_kernel<kGeluBf16>), grid, dim3(256), 0, stream, set, x, M, N, K);
      break;
  }
  return hipGetLastError();
}

}  // namespace rkv
