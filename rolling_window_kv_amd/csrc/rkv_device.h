// Device-side helpers shared by the rkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rkv.h"

namespace rkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// bfloat16 bit pattern -> float (exact).
__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }

// float -> bfloat16 bit pattern, round to nearest, ties to even.
// NaN maps to a quiet NaN; overflow rounds to infinity like IEEE RNE.
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float rne_bf16f(float f) { return bf2f(f2bf(f)); }

// Two floats -> packed bfloat16 pair (low half = a), round to nearest even,
// with gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t cvt2_bf16(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, b2));
}

// float64 -> float32 that rounds to the same bfloat16 as the float64 value
// would directly (nearest, ties to even).  Rounding to float32 first is exact
// for this purpose unless the float32 result lands exactly on a bfloat16 tie;
// then it is moved one float32 step toward the float64 value (or kept when
// the float64 value is the tie itself).
__device__ __forceinline__ float f64_for_bf16(double y) {
  const float t = (float)y;
  uint32_t u = __float_as_uint(t);
  if ((u & 0xffffu) == 0x8000u) {
    const double back = (double)t;
    if (back != y) u = fabs(y) > fabs(back) ? u + 1u : u - 1u;
  }
  return __uint_as_float(u);
}

// float64 pair -> packed, correctly rounded bfloat16 pair.
__device__ __forceinline__ uint32_t cvt2_bf16_f64(double a, double b) {
  return cvt2_bf16(f64_for_bf16(a), f64_for_bf16(b));
}

// float64 -> bfloat16 bit pattern, correctly rounded (single value).
__device__ __forceinline__ uint32_t f64_to_bf16(double y) {
  return f2bf(f64_for_bf16(y));
}

// Rotation of one pair in float64: y1 = x1 c - x2 s, y2 = x1 s + x2 c.
__device__ __forceinline__ void rotate_pair64(double x1, double x2, double c, double s,
                                              double& y1, double& y2) {
  y1 = fma(x1, c, -(x2 * s));
  y2 = fma(x1, s, x2 * c);
}

// Element e (0..7) of 8 bfloat16 values packed in a 16-byte vector.
__device__ __forceinline__ uint32_t elem8(const u32x4& w, int e) {
  return (w[e >> 1] >> (16 * (e & 1))) & 0xffffu;
}

// Unpack / pack 8 bfloat16 values held in a 16-byte vector.
__device__ __forceinline__ void unpack8(const u32x4& w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf2f(w[i] & 0xffffu);
    f[2 * i + 1] = bf2f(w[i] >> 16);
  }
}

__device__ __forceinline__ u32x4 pack8(const float* f) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = f2bf(f[2 * i]) | (f2bf(f[2 * i + 1]) << 16);
  return w;
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(uint16_t* p, const u32x4& w) {
  *reinterpret_cast<u32x4*>(p) = w;
}
__device__ __forceinline__ u32x2 ld8(const uint16_t* p) {
  return *reinterpret_cast<const u32x2*>(p);
}
__device__ __forceinline__ void st8(uint16_t* p, const u32x2& w) {
  *reinterpret_cast<u32x2*>(p) = w;
}

// Address of row r of (layer, stream, head) in a cache tensor.
struct KvAddr {
  int64_t ls, ss, hs, rs;
  __device__ __forceinline__ int64_t base(int l, int s, int g) const {
    return (int64_t)l * ls + (int64_t)s * ss + (int64_t)g * hs;
  }
};

}  // namespace rkv
