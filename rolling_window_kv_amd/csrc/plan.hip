// Step plan kernel: advance every stream's cache state by one clock step
// (the per-mode rules are in rkv_plan.h).  One wave of 64 threads per stream.

#include "rkv_device.h"
#include "rkv_internal.h"
#include "rkv_plan.h"

namespace rkv {
namespace {

__global__ __launch_bounds__(64) void advance_kernel(rkv_stream_state* __restrict__ st,
                                                     rkv_step_plan* __restrict__ plan, int mode,
                                                     int dc, int F, int half, Theta th) {
  advance_stream(st, plan, blockIdx.x, threadIdx.x, mode, dc, F, half, th);
}

}  // namespace

hipError_t launch_advance(const rkv_cfg* cfg, rkv_stream_state* st, rkv_step_plan* plan,
                          hipStream_t stream) {
  hipLaunchKernelGGL(advance_kernel, dim3(cfg->num_streams), dim3(64), 0, stream, st, plan,
                     cfg->mode, cfg->rebase_chunk, cfg->new_rows, cfg->head_dim / 2,
                     theta_table(cfg));
  return hipGetLastError();
}

}  // namespace rkv
