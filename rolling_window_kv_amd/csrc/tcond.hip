// Delay conditioning (Audio8 ASR Infinite explainer, 可配置转写延迟): the
// delay count as a sinusoidal embedding plus a frame-length table row forms
// t_cond, and each decoder layer's attention output is scaled and shifted
// feature-wise by [gamma_l; beta_l] = A_l t_cond (the form of the modulation
// is not given by the sources; this is the reading the C ABI states).
//
// The modulation vectors depend only on the setting and the layer, so they
// are computed once per change of setting (prepare_kernel: one workgroup per
// (layer, condition), t_cond in LDS, one wave per output row, its products
// summed across the lanes).  The per-step work is the elementwise
// modulate_kernel: one workgroup per (layer, stream) row, 8 features per
// thread, the vectors of a condition read from L2 by every stream using it.

#include <math.h>

#include "rkv_device.h"
#include "rkv_tcond.h"

namespace rkv {
namespace {

constexpr int kTcondThreads = 256;

__global__ __launch_bounds__(kTcondThreads) void prepare_kernel(
    TcondConds conds, const uint16_t* __restrict__ table, const uint16_t* __restrict__ weights,
    float* __restrict__ mod, int hidden, int dim, int num_conds) {
  __shared__ float tc[RKV_TCOND_MAX_DIM];
  const int l = blockIdx.x, c = blockIdx.y;
  const int half = dim >> 1;
  const double n = (double)conds.num_delay[c];
  const uint16_t* row = table + (int64_t)conds.frame_len[c] * dim;
  for (int i = threadIdx.x; i < half; i += kTcondThreads) {
    const double w = pow(10000.0, -(double)i / (double)half);
    double sn, cs;
    sincos(n * w, &sn, &cs);
    tc[i] = (float)sn + bf2f(row[i]);
    tc[half + i] = (float)cs + bf2f(row[half + i]);
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint16_t* A = weights + (int64_t)l * 2 * hidden * dim;
  float* out = mod + ((int64_t)l * num_conds + c) * 2 * hidden;
  for (int r = wave; r < 2 * hidden; r += kTcondThreads / 64) {
    const uint16_t* ar = A + (int64_t)r * dim;
    float acc = 0.f;
    for (int i = lane; i < dim; i += 64) acc = fmaf(bf2f(ar[i]), tc[i], acc);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) out[r] = acc;
  }
}

template <bool F32>
__global__ __launch_bounds__(kTcondThreads) void modulate_kernel(
    const float* __restrict__ mod, const int32_t* __restrict__ stream_cond, void* __restrict__ out,
    int streams, int hidden, int num_conds) {
  const int row = blockIdx.x;                  // layer * streams + stream
  const int l = row / streams, s = row - l * streams;
  const int c = stream_cond[s];
  if (c < 0 || c >= num_conds) return;         // conditioning off for this stream
  const float* g = mod + ((int64_t)l * num_conds + c) * 2 * hidden;
  const float* b = g + hidden;
  for (int j = 8 * threadIdx.x; j < hidden; j += 8 * kTcondThreads) {
    float gg[8], bb[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 gv = *reinterpret_cast<const f32x4*>(g + j + 4 * h);
      const f32x4 bv = *reinterpret_cast<const f32x4*>(b + j + 4 * h);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        gg[4 * h + k] = 1.0f + gv[k];
        bb[4 * h + k] = bv[k];
      }
    }
    if (F32) {
      float* o = reinterpret_cast<float*>(out) + (int64_t)row * hidden + j;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 v = *reinterpret_cast<const f32x4*>(o + 4 * h);
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = fmaf(v[k], gg[4 * h + k], bb[4 * h + k]);
        *reinterpret_cast<f32x4*>(o + 4 * h) = v;
      }
    } else {
      uint16_t* o = reinterpret_cast<uint16_t*>(out) + (int64_t)row * hidden + j;
      float f[8];
      unpack8(ld16(o), f);
#pragma unroll
      for (int k = 0; k < 8; ++k) f[k] = fmaf(f[k], gg[k], bb[k]);
      st16(o, pack8(f));
    }
  }
}

}  // namespace

hipError_t launch_tcond_prepare(const rkv_tcond_cfg* tc, const TcondConds& conds,
                                const uint16_t* table, const uint16_t* weights, float* mod,
                                hipStream_t stream) {
  hipLaunchKernelGGL(prepare_kernel, dim3(tc->num_layers, tc->num_conds), dim3(kTcondThreads), 0,
                     stream, conds, table, weights, mod, tc->hidden, tc->dim, tc->num_conds);
  return hipGetLastError();
}

hipError_t launch_tcond_modulate(int layers, int streams, int hidden, int num_conds, bool out_f32,
                                 const float* mod, const int32_t* stream_cond, void* out,
                                 hipStream_t stream) {
  const dim3 grid((unsigned)layers * (unsigned)streams), block(kTcondThreads);
  if (out_f32)
    hipLaunchKernelGGL(modulate_kernel<true>, grid, block, 0, stream, mod, stream_cond, out,
                       streams, hidden, num_conds);
  else
    hipLaunchKernelGGL(modulate_kernel<false>, grid, block, 0, stream, mod, stream_cond, out,
                       streams, hidden, num_conds);
  return hipGetLastError();
}

}  // namespace rkv
