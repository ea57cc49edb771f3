// Host <-> kernel interface of the device-side expert streaming (k_stream.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moeq {

// per expert up to 9 segments (codes, scales, biases of gate, up, down), each
// a stack of per-expert blocks of `bytes`
constexpr int kMaxStreamExperts = 1024;
constexpr int kMaxStreamSlots = 1024;
struct StreamCopy {
  const char* src[9];   // device-mapped addresses of the pinned host stacks
  char* dst[9];         // the slot stacks
  uint64_t bytes[9];    // per-expert bytes of each segment
  int nseg;
  int parts;            // blocks per copied expert
};
int launch_stream_experts(const StreamCopy& P, const int32_t* idx, int MK, int E, int S,
                          int32_t* slot_expert, int64_t* slot_stamp, int32_t* slot_idx,
                          int32_t* list, int32_t* n_copied, hipStream_t s);

}  // namespace moeq
