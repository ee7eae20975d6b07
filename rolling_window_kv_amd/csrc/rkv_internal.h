// Host-side launch interfaces between the C entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rkv.h"
#include "rkv_plan.h"

namespace rkv {

struct RingArgs {
  uint16_t* k;
  uint16_t* v;
  uint16_t* klo;
  int64_t ls, ss, hs, rs;  // layer / stream / head / slot strides (elements)
  int32_t slots;
};

struct AttnArgs {
  const rkv_step_plan* plan;
  RingArgs ring;
  const uint16_t* q;
  const uint16_t* knew;
  const uint16_t* vnew;
  void* out;
  float* ws;          // split partials (nsplit > 1)
  // One counter per item (nsplit > 1): the split that takes the last ticket
  // merges the item's partials in this launch and returns the counter to 0.
  // Null: the partials are merged by a second launch (combine_kernel).
  uint32_t* tickets;
  int32_t S, L, Hkv;  // streams, layers, KV heads (ENC: heads)
  int32_t G;          // query vectors per KV head (decoder: Hq/Hkv; ENC: F)
  int32_t F;          // frames per chunk (ENC), 1 otherwise
  int32_t nsplit;
  int32_t out_f32;
  float scale_log2;   // softmax scale * log2(e)
  // Pipelined decode step: extra waves of the same launch compute the next
  // step's plan into adv_plan and advance adv_state (null: none).
  rkv_stream_state* adv_state;
  rkv_step_plan* adv_plan;
  int32_t adv_mode, adv_dc, adv_F, adv_half;
  // Encoder chunks: pull_blocks extra workgroups, dispatched after the
  // attention's, read [pull, pull + pull_bytes) into the cache (the next
  // products' weights of an encoder step); null: none.
  const char* pull;
  int64_t pull_bytes;
  int32_t pull_blocks;
  // Decoder: delay conditioning applied to the output as it is stored, with
  // exactly the arithmetic of rkv_tcond_modulate on the stored value:
  // out <- out (1 + gamma) + beta, the vectors of condition tc_cond[s] of
  // tc_mod [L][tc_conds][2][Hq d]; null: none.
  const float* tc_mod;
  const int32_t* tc_cond;
  int32_t tc_conds;
  Theta adv_theta;
};

// Modulation vector (gamma; beta follows `hidden` floats later) of a stream's
// condition for one layer, or null when the stream's condition is off.
__device__ __forceinline__ const float* tcond_row(const AttnArgs& a, int l, int s, int hidden) {
  if (!a.tc_mod) return nullptr;
  const int c = a.tc_cond[s];
  if (c < 0 || c >= a.tc_conds) return nullptr;
  return a.tc_mod + ((int64_t)l * a.tc_conds + c) * 2 * hidden;
}

enum AttnKind { kDecodeRead = 0, kDecodeFused = 1, kEncoderFused = 2 };

// Number of key-range splits for an attention call.
int choose_splits(const rkv_cfg* cfg, int32_t slots);
// Split launches of at most this many workgroups merge their splits in the
// same launch: one round of resident 4-wave workgroups on 256 CUs (3 per CU).
constexpr int64_t kMergeInLaunchMaxBlocks = 768;
// Floats of workspace per (item, split) partial.
__host__ __device__ inline int64_t partial_floats(int d) { return 16 + 8 * (int64_t)d; }

hipError_t launch_advance(const rkv_cfg* cfg, rkv_stream_state* st, rkv_step_plan* plan,
                          hipStream_t stream);

// Streams restarted by one reset launch (passed by value in kernel arguments).
struct ResetList {
  static constexpr int kMax = 64;
  int32_t n;
  int32_t stream[kMax];
  int64_t origin[kMax];
};
hipError_t launch_reset(const rkv_cfg* cfg, rkv_stream_state* st, rkv_step_plan* plan,
                        const ResetList& list, hipStream_t stream);
hipError_t launch_append(const rkv_cfg* cfg, const rkv_step_plan* plan, const RingArgs& ring,
                         const uint16_t* knew, const uint16_t* vnew, hipStream_t stream);
hipError_t launch_rebase(const rkv_cfg* cfg, const rkv_step_plan* plan, const RingArgs& ring,
                         hipStream_t stream);
hipError_t launch_compact(const rkv_cfg* cfg, const rkv_step_plan* plan, const RingArgs& ring,
                          hipStream_t stream);
hipError_t launch_attention(const rkv_cfg* cfg, AttnKind kind, const AttnArgs& args,
                            hipStream_t stream);

}  // namespace rkv
