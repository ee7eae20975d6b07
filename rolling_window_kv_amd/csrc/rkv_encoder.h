// Launchers of the encoder-stack building blocks (encoder.hip), sequenced by
// rkv_encoder_step in the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rkv {

enum class GemmEpilogue { kStoreBf16 = 0, kAddF32 = 1, kGeluBf16 = 2, kStoreF32 = 3 };

// Products launched together by one launch_gemm (q/k/v, or k-slices).
constexpr int kGemmMaxSet = 4;

// Largest hidden width the encoder kernels take: the RMSNorm keeps a row in
// registers, kNormPerThread float4 per thread of a kNormThreads workgroup.
constexpr int kNormThreads = 256;
constexpr int kNormPerThread = 4;
constexpr int kEncoderMaxHidden = 4 * kNormThreads * kNormPerThread;

// x[m] += parts[0][m] + ... + parts[nparts-1][m] (in that order, parts[p] at
// parts + p * part_stride; nparts 0, 1, 2 or 4; 0 leaves x), then, unless a
// is null, a[m] = bfloat16(x[m] / sqrt(mean(x[m]^2) + eps) * g); x float32
// [M][hidden],
// hidden a multiple of 4, at most kEncoderMaxHidden.
hipError_t launch_rmsnorm(float* x, const float* parts, int nparts, int64_t part_stride,
                          const uint16_t* g, uint16_t* a, int M, int hidden, float eps,
                          hipStream_t stream);

// For i < count (<= kGemmMaxSet): C_i[m][n] = sum_{k < K} x_i[m][k] w_i[n][k]
// (bfloat16 operands with row stride ld, float32 sums), stored as bfloat16,
// added to a float32 C_i, stored as bfloat16 gelu(.), or stored as float32.
// N a multiple of 64, K a multiple of 64.
hipError_t launch_gemm(GemmEpilogue ep, const uint16_t* const* w, const uint16_t* const* x,
                       void* const* c, int count, int M, int N, int K, int ld,
                       hipStream_t stream);

}  // namespace rkv
