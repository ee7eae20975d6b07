// Launchers of the encoder-stack building blocks (encoder.hip), sequenced by
// rkv_encoder_step in the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rkv {

enum class GemmEpilogue { kStoreBf16 = 0, kAddF32 = 1, kGeluBf16 = 2 };

// a[m] = bfloat16(x[m] / sqrt(mean(x[m]^2) + eps) * g), x float32 [M][hidden].
hipError_t launch_rmsnorm(const float* x, const uint16_t* g, uint16_t* a, int M, int hidden,
                          float eps, hipStream_t stream);

// For i < count (<= 3): C_i[m][n] = sum_k x[m][k] w_i[n][k] (bfloat16 operands,
// float32 sums), stored as bfloat16, added to a float32 C_i, or stored as
// bfloat16 gelu(.).  N a multiple of 32, K a multiple of 32.
hipError_t launch_gemm(GemmEpilogue ep, const uint16_t* const* w, void* const* c, int count,
                       const uint16_t* x, int M, int N, int K, hipStream_t stream);

}  // namespace rkv
