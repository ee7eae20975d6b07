// Rolling log-mel front end (voxtral.c explainer, section 三: even the mel
// buffer rolls -- samples that can no longer reach a future frame are
// dropped -- so the whole pipeline runs in bounded memory).  Features as the
// Audio8 explainer's file table gives them: 16 kHz audio, 128 mel bands, hop
// 160; a step of the 80 ms clock carries 1280 samples.
//
// Per stream the only state between steps is the tail of n_fft - hop
// samples: frame f of a step covers samples [f*hop, f*hop + n_fft) of
// tail ++ new samples, so every frame is causal and a step of n samples
// yields n / hop frames.  One workgroup per (stream, frame): the windowed
// frame and a twiddle table sit in LDS, two threads per DFT bin sum the real
// DFT in float32 (its twiddles by rotation, see below), and a thread per mel
// band applies its filter row and the log.  The new tail is the last n_fft - hop new samples (the step carries
// at least that many), written to a second buffer so that no workgroup reads
// a tail another one has replaced.

#include <math.h>

#include "rkv_device.h"
#include "rkv_internal.h"
#include "rkv_mel.h"

namespace rkv {
namespace {

constexpr int kMelThreads = 512;
constexpr int kMelParts = 2;       // lanes per DFT bin (a power of 2 dividing 64)
constexpr int kMelResync = 64;     // samples between twiddles taken from the table

__global__ __launch_bounds__(kMelThreads) void mel_kernel(
    const float* __restrict__ tail_in, float* __restrict__ tail_out,
    const float* __restrict__ samples, const float* __restrict__ filters,
    float* __restrict__ out, int n_fft, int hop, int n_mels, int per_step) {
  __shared__ float sx[RKV_MEL_MAX_FFT];        // windowed frame
  __shared__ float scos[RKV_MEL_MAX_FFT];      // cos(2 pi m / n_fft)
  __shared__ float ssin[RKV_MEL_MAX_FFT];      // sin(2 pi m / n_fft)
  __shared__ float spow[RKV_MEL_MAX_FFT / 2 + 1];
  const int s = blockIdx.x;
  const int f = blockIdx.y;
  const int keep = n_fft - hop;
  const float* tin = tail_in + (int64_t)s * keep;
  const float* xin = samples + (int64_t)s * per_step;
  for (int n = threadIdx.x; n < n_fft; n += kMelThreads) {
    const int i = f * hop + n;                           // index into tail ++ samples
    const float x = i < keep ? tin[i] : xin[i - keep];
    double sn, cs;
    sincospi(2.0 * (double)n / (double)n_fft, &sn, &cs);
    scos[n] = (float)cs;
    ssin[n] = (float)sn;
    sx[n] = x * (float)(0.5 - 0.5 * cs);                 // periodic Hann window
  }
  if (f == 0) {                                          // the tail the next step needs
    for (int n = threadIdx.x; n < keep; n += kMelThreads)
      tail_out[(int64_t)s * keep + n] = xin[per_step - keep + n];
  }
  __syncthreads();
  // Bin k's twiddles cos/sin(2 pi k n / n_fft) advance by a rotation through
  // 2 pi k / n_fft per sample, restarted from the table every kMelResync
  // samples (so the float32 recurrence drifts by at most that many
  // roundings).  Reading the table at k n mod n_fft for every sample would put
  // the lanes of a wave n entries apart in LDS: bank conflicts for most n.
  // kMelParts adjacent lanes share a bin, one part of the frame each, and
  // add their sums with shuffles.
  const int bins = n_fft / 2 + 1;
  const int part = (n_fft + kMelParts - 1) / kMelParts;
  for (int u = threadIdx.x; u < kMelParts * bins; u += kMelThreads) {
    const int k = u / kMelParts, h = u % kMelParts;
    const float cw = scos[k], sw = ssin[k];
    float re = 0.f, im = 0.f;
    const int nb = h * part, ne = min(n_fft, nb + part);
    for (int n0 = nb; n0 < ne; n0 += kMelResync) {
      const int m0 = (int)(((int64_t)k * n0) % n_fft);
      float tc = scos[m0], ts = ssin[m0];
      const int n1 = min(n0 + kMelResync, ne);
      for (int n = n0; n < n1; ++n) {
        const float x = sx[n];
        re = fmaf(x, tc, re);
        im = fmaf(x, ts, im);
        const float nc = fmaf(tc, cw, -ts * sw);
        ts = fmaf(tc, sw, ts * cw);
        tc = nc;
      }
    }
#pragma unroll
    for (int off = 1; off < kMelParts; off <<= 1) {
      re += __shfl_xor(re, off);
      im += __shfl_xor(im, off);
    }
    if (h == 0) spow[k] = fmaf(re, re, im * im);
  }
  __syncthreads();
  float* o = out + ((int64_t)s * (per_step / hop) + f) * n_mels;
  for (int b = threadIdx.x; b < n_mels; b += kMelThreads) {
    const float* w = filters + (int64_t)b * bins;
    float e = 0.f;
    for (int k = 0; k < bins; ++k) e = fmaf(w[k], spow[k], e);
    o[b] = log10f(fmaxf(e, 1e-10f));
  }
}

}  // namespace

hipError_t launch_mel(const rkv_mel_cfg* c, const float* tail_in, float* tail_out,
                      const float* samples, const float* filters, float* out,
                      hipStream_t stream) {
  const dim3 grid(c->num_streams, c->samples_per_step / c->hop);
  hipLaunchKernelGGL(mel_kernel, grid, dim3(kMelThreads), 0, stream, tail_in, tail_out, samples,
                     filters, out, c->n_fft, c->hop, c->n_mels, c->samples_per_step);
  return hipGetLastError();
}

}  // namespace rkv
