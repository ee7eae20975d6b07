// Launchers of the delay-conditioning kernels (tcond.hip), called by the C
// entry points after validation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rkv.h"

namespace rkv {

// Delay counts and frame-length rows of the conditions (passed by value).
struct TcondConds {
  int32_t num_delay[RKV_TCOND_MAX_CONDS];
  int32_t frame_len[RKV_TCOND_MAX_CONDS];
};

hipError_t launch_tcond_prepare(const rkv_tcond_cfg* tc, const TcondConds& conds,
                                const uint16_t* table, const uint16_t* weights, float* mod,
                                hipStream_t stream);

hipError_t launch_tcond_modulate(int layers, int streams, int hidden, int num_conds, bool out_f32,
                                 const float* mod, const int32_t* stream_cond, void* out,
                                 hipStream_t stream);

}  // namespace rkv
