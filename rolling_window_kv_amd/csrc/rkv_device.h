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

// float64 -> float32 rounded to odd: truncated toward zero, with the last bit
// set when the conversion is inexact.  Rounding that float32 to nearest in a
// format of at most 22 significant bits gives the correctly rounded float64
// value (the sticky bit keeps the float64 value's side of every tie).
__device__ __forceinline__ float f64_to_f32_odd(double y) {
  const float t = (float)y;
  const double back = (double)t;
  if (back == y) return t;
  uint32_t u = __float_as_uint(t);
  if (fabs(back) > fabs(y)) u -= 1u;   // rounded away from zero: one step back
  return __uint_as_float(u | 1u);
}

// Storage formats of the cache's 16-bit words (K, V, the K residual):
// bfloat16, or IEEE binary16 for the fp16 cache variant (voxtral.c explainer,
// section 七).  to_f widens a stored word; cvt2 rounds two floats to nearest
// (ties to even) and packs them (low half = a); cvt2_f64 / from_f64 round
// float64 values correctly; from_bf16x2 converts two packed bfloat16 inputs.
struct StoreBf16 {
  static __device__ __forceinline__ float to_f(uint32_t h) { return bf2f(h); }
  static __device__ __forceinline__ uint32_t cvt2(float a, float b) { return cvt2_bf16(a, b); }
  static __device__ __forceinline__ uint32_t cvt2_f64(double a, double b) {
    return cvt2_bf16_f64(a, b);
  }
  static __device__ __forceinline__ uint32_t from_f64(double y) { return f64_to_bf16(y); }
  static __device__ __forceinline__ uint32_t from_bf16x2(uint32_t w) { return w; }
};

struct StoreF16 {
  static __device__ __forceinline__ float to_f(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  }
  static __device__ __forceinline__ uint32_t cvt2(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, h2));
  }
  static __device__ __forceinline__ uint32_t cvt2_f64(double a, double b) {
    return cvt2(f64_to_f32_odd(a), f64_to_f32_odd(b));
  }
  static __device__ __forceinline__ uint32_t from_f64(double y) {
    return cvt2(f64_to_f32_odd(y), 0.f) & 0xffffu;
  }
  static __device__ __forceinline__ uint32_t from_bf16x2(uint32_t w) {
    return cvt2(bf2f(w & 0xffffu), bf2f(w >> 16));
  }
};

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

// Rotation of one pair by an angle whose cosine and sine are given as float32
// hi + lo pairs (c = ch + cl, s = sh + sl): y1 = x1 c - x2 s, y2 = x1 s + x2 c
// for float32 inputs x1, x2 with at most 16 significant bits.  The rounding
// error of each large product is recovered exactly with an fma and added back
// with the small terms, so the error is about 2^-24 of the result itself
// rather than of the products: under cancellation the result keeps its
// accuracy, and rounding it to bfloat16 lands within 1 ulp of the correctly
// rounded rotation.
__device__ __forceinline__ void rotate_pair_ff(float x1, float x2, float ch, float cl, float sh,
                                               float sl, float& y1, float& y2) {
  const float p1 = x2 * sh;
  const float e1 = fmaf(x2, sh, -p1);             // x2 sh = p1 + e1 exactly
  const float h1 = fmaf(x1, ch, -p1);             // x1 ch - p1, rounded once
  const float t1 = fmaf(x1, cl, -fmaf(x2, sl, e1));
  y1 = h1 + t1;
  const float p2 = x2 * ch;
  const float e2 = fmaf(x2, ch, -p2);             // x2 ch = p2 + e2 exactly
  const float h2 = fmaf(x1, sh, p2);              // x1 sh + p2, rounded once
  const float t2 = fmaf(x1, sl, fmaf(x2, cl, e2));
  y2 = h2 + t2;
}

// Re-base one chunk pair of a K row by R(-D): a holds dims i0 .. i0+7 and b
// dims i0 + d/2 .. (the rotary partners); table(e) returns {ch, cl, sh, sl} of
// pair i0 + e, the float32 hi/lo split of cos(D theta) and -sin(D theta).
// Inputs are exact in float32 (one stored word, or hi + lo with at most 22
// significant bits); each result is rounded to nearest in the storage format
// SF.  Compensated: la / lb hold the residuals; x = hi + lo is rotated and
// split again into hi and lo.
template <bool COMP, typename SF, typename Table>
__device__ __forceinline__ void rebase_chunks_ff(u32x4& a, u32x4& b, u32x4& la, u32x4& lb,
                                                 Table table) {
  u32x4 na, nb, nla, nlb;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float y1[2], y2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = 2 * w + h;
      const int sh = 16 * h;
      float x1 = SF::to_f((a[w] >> sh) & 0xffffu);
      float x2 = SF::to_f((b[w] >> sh) & 0xffffu);
      if (COMP) {
        x1 += SF::to_f((la[w] >> sh) & 0xffffu);
        x2 += SF::to_f((lb[w] >> sh) & 0xffffu);
      }
      const f32x4 t = table(e);
      rotate_pair_ff(x1, x2, t[0], t[1], t[2], t[3], y1[h], y2[h]);
    }
    na[w] = SF::cvt2(y1[0], y1[1]);
    nb[w] = SF::cvt2(y2[0], y2[1]);
    if (COMP) {
      nla[w] = SF::cvt2(y1[0] - SF::to_f(na[w] & 0xffffu), y1[1] - SF::to_f(na[w] >> 16));
      nlb[w] = SF::cvt2(y2[0] - SF::to_f(nb[w] & 0xffffu), y2[1] - SF::to_f(nb[w] >> 16));
    }
  }
  a = na;
  b = nb;
  if (COMP) {
    la = nla;
    lb = nlb;
  }
}

// {ch, cl, sh, sl}: float32 hi/lo split of c = cos(x) and -s = -sin(x) for
// rebase_chunks_ff.
__device__ __forceinline__ f32x4 rebase_table_entry(double c, double s) {
  const float ch = (float)c;
  const float sh = (float)(-s);
  return f32x4{ch, (float)(c - (double)ch), sh, (float)(-s - (double)sh)};
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
// Streaming (non-temporal) loads, for data read once per launch where each
// instruction covers whole 128-byte lines (V rows: 16 lanes span a row).
// Measured: V tiles loaded this way cut the decode launch by ~5 % at 36 x 64;
// K tiles, whose instructions cover half lines, got slower with the hint.
__device__ __forceinline__ u32x4 ld16_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x2 ld8_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

// Device-scope accesses for data that one workgroup hands to another within a
// launch.  The eight XCDs' L2 caches are not coherent with each other, and an
// agent-scope release/acquire makes them so by writing back and invalidating
// the whole L2 -- in the middle of a launch that streams the cache through it.
// Instead only the handed-over words use the device-scope cache policy (sc1):
// such a store writes through to memory, such a load is not served from a
// possibly stale L1 or L2 copy (the accesses an agent-scope relaxed atomic
// load or store compiles to).  Order comes from waiting for the stores to
// complete (wait_stores) before the hand-over's atomic counter.
constexpr int kDeviceScope = 16;  // buffer cache-policy operand: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_buffer(const void* p, uint32_t bytes) {
  // word 3: the gfx9 family's raw-buffer format (32-bit data, untyped access)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ void st_dev(__amdgpu_buffer_rsrc_t r, int byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, byte_off, 0, kDeviceScope);
}
__device__ __forceinline__ void st_dev4(__amdgpu_buffer_rsrc_t r, int byte_off, const f32x4& v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, byte_off, 0,
                                         kDeviceScope);
}
__device__ __forceinline__ float ld_dev(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, kDeviceScope));
}
__device__ __forceinline__ f32x4 ld_dev4(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(f32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kDeviceScope));
}
// Wait until every store this wave issued has completed (and keep the
// compiler from moving memory accesses across the wait).
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 16 bytes per lane from global memory into LDS (global_load_lds_dwordx4):
// lane i of the wave writes l + 16 i bytes, l being the same for every lane.
__device__ __forceinline__ void lds_dma16(const uint16_t* g, uint16_t* l) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)l, 16, 0, 0);
}

// Reads [p, p + bytes) once, 1 KB per wave instruction, into one scratch KB of
// LDS (every wave overwrites the same bytes), so that the lines are in the
// infinity cache when a later launch reads them; workgroup wg of nwg.  The
// data goes nowhere else; a wave's end waits for its loads.
__device__ __forceinline__ void pull_into_cache(const char* p, int64_t bytes, int wg, int nwg,
                                                uint16_t* lds_scratch_1kb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int64_t last = bytes - 16;
  for (int64_t off = ((int64_t)wg * nw + wave) * 1024; off < bytes;
       off += (int64_t)nwg * nw * 1024) {
    int64_t o = off + 16 * lane;
    o = o < last ? o : last;
    lds_dma16(reinterpret_cast<const uint16_t*>(p + o), lds_scratch_1kb);
  }
}

// Address of row r of (layer, stream, head) in a cache tensor.
struct KvAddr {
  int64_t ls, ss, hs, rs;
  __device__ __forceinline__ int64_t base(int l, int s, int g) const {
    return (int64_t)l * ls + (int64_t)s * ss + (int64_t)g * hs;
  }
};

}  // namespace rkv
