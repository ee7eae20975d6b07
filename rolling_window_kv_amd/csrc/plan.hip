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

// Continuous-mode restart of the listed streams (voxtral.c explainer,
// section 四: a hard decoder reset, no context kept): one wave per listed
// stream builds the stream's initial state at the new origin with its window
// and capacity; with a plan, the wave also advances that state by the step
// whose plan was already written.  Lists are applied in order: the host
// splits them so no stream appears twice in one launch.
__global__ __launch_bounds__(64) void reset_kernel(rkv_stream_state* __restrict__ st,
                                                   rkv_step_plan* __restrict__ plan,
                                                   ResetList list, int mode, int dc, int F,
                                                   int half, Theta th) {
  const int i = blockIdx.x;
  const int s = list.stream[i];
  const rkv_stream_state old = st[s];
  const rkv_stream_state x = initial_state(list.origin[i], old.window, old.cap, mode, dc);
  if (plan) {
    advance_from(x, st, plan, s, threadIdx.x, mode, dc, F, half, th);
  } else if (threadIdx.x == 0) {
    st[s] = x;
  }
}

}  // namespace

hipError_t launch_reset(const rkv_cfg* cfg, rkv_stream_state* st, rkv_step_plan* plan,
                        const ResetList& list, hipStream_t stream) {
  if (list.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(reset_kernel, dim3(list.n), dim3(64), 0, stream, st, plan, list, cfg->mode,
                     cfg->rebase_chunk, cfg->new_rows, cfg->head_dim / 2, theta_table(cfg));
  return hipGetLastError();
}

hipError_t launch_advance(const rkv_cfg* cfg, rkv_stream_state* st, rkv_step_plan* plan,
                          hipStream_t stream) {
  hipLaunchKernelGGL(advance_kernel, dim3(cfg->num_streams), dim3(64), 0, stream, st, plan,
                     cfg->mode, cfg->rebase_chunk, cfg->new_rows, cfg->head_dim / 2,
                     theta_table(cfg));
  return hipGetLastError();
}

}  // namespace rkv
