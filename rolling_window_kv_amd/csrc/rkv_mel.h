// Launcher of the rolling log-mel front end (mel.hip), called by the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include "rkv.h"

namespace rkv {

hipError_t launch_mel(const rkv_mel_cfg* c, const float* tail_in, float* tail_out,
                      const float* samples, const float* filters, float* out,
                      hipStream_t stream);

}  // namespace rkv
