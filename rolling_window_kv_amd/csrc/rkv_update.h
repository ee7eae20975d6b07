// Launcher of the combined re-base + append of one step (update.hip), called
// by rkv_update_step after validation.
#pragma once

#include "rkv_internal.h"

namespace rkv {

hipError_t launch_update(const rkv_cfg* cfg, const rkv_step_plan* plan, const RingArgs& ring,
                         const uint16_t* knew, const uint16_t* vnew, hipStream_t stream);

}  // namespace rkv
