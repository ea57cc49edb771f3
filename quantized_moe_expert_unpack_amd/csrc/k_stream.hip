// Device-side expert streaming: the slot choice (an LRU over S device slots)
// and the host->device copies of the missing experts, with no host round
// trip between the routing and the forward.
//
// flash-moe-inference skill page, parallel expert loading: K expert reads per
// layer into expert buffers, the OS page cache acting as the LRU.  Here the
// experts sit in pinned host memory mapped into the device's address space,
// the buffers are HBM slots, and the copy is one kernel whose waves read the
// host stacks over PCIe directly (no copy engine call per tensor).
//
// k_slot_lru (one wave) takes the same decisions as the host-side LRU of
// moe_stream_experts: the call's distinct experts in order of first
// appearance; experts already in a slot keep it and are stamped with the
// call's number first; every other one takes the lowest empty slot not
// stamped by this call, else the slot with the oldest stamp (lowest slot on
// a tie).  It writes the slot of every pair and a copy list (count, then
// (expert, slot) pairs) that k_slot_copy reads.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"
#include "launch.h"
#include "stream.h"

namespace moeq {
namespace {

constexpr int kLruThreads = 64;      // one wave
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;       // 16-byte loads in flight per thread

__global__ __launch_bounds__(kLruThreads) void k_slot_lru(const int32_t* __restrict__ idx, int MK, int E,
                                                          int S, int32_t* __restrict__ slot_expert,
                                                          int64_t* __restrict__ slot_stamp,
                                                          int32_t* __restrict__ slot_idx,
                                                          int32_t* __restrict__ list,
                                                          int32_t* __restrict__ n_copied) {
  __shared__ int where[kMaxStreamExperts];      // expert -> slot (-1 unused, -2 needed)
  __shared__ int s_exp[kMaxStreamSlots];
  __shared__ int64_t s_stamp[kMaxStreamSlots];
  __shared__ int need[kMaxStreamSlots];
  __shared__ int s_n;
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += kLruThreads) where[e] = -1;
  for (int s = lane; s < S; s += kLruThreads) {
    s_exp[s] = slot_expert[s];
    s_stamp[s] = slot_stamp[s];
  }
  __syncthreads();
  // distinct valid experts in order of first appearance (MK <= S pairs)
  if (lane == 0) {
    int n = 0;
    for (int i = 0; i < MK; ++i) {
      const int e = idx[i];
      if (e < 0 || e >= E || where[e] == -2) continue;
      where[e] = -2;
      need[n++] = e;
    }
    s_n = n;
  }
  __syncthreads();
  const int64_t now = slot_stamp[S] + 1;
  // hits: a slot holding a needed expert keeps it (each expert is in at most
  // one slot)
  for (int s = lane; s < S; s += kLruThreads) {
    const int e = s_exp[s];
    if (e >= 0 && e < E && where[e] == -2) {
      where[e] = s;
      s_stamp[s] = now;
    }
  }
  __syncthreads();
  const int n = s_n;
  int copies = 0;
  for (int j = 0; j < n; ++j) {
    const int e = need[j];
    if (where[e] >= 0) continue;                 // uniform: LDS read by every lane
    // victim key: an empty slot sorts below every occupied one; occupied
    // slots by (stamp, slot); slots stamped by this call are not candidates
    uint64_t best = ~0ull;
    for (int s = lane; s < S; s += kLruThreads) {
      if (s_stamp[s] == now) continue;
      const uint64_t key = s_exp[s] < 0 ? (uint64_t)s
                                        : (((uint64_t)s_stamp[s] + 1) << 12) | (uint64_t)s;
      best = key < best ? key : best;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const uint64_t other = __shfl_xor(best, o, kLruThreads);
      best = other < best ? other : best;
    }
    // a candidate exists while the state is the library's own (at most
    // MK <= S distinct experts, fewer stamped so far); if it was altered and
    // none is left, the expert gets no slot and its pairs slot S
    if (best == ~0ull) continue;
    const int v = (int)(best & 0xFFF);
    if (lane == 0) {
      s_exp[v] = e;
      s_stamp[v] = now;
      where[e] = v;
      list[1 + 2 * copies] = e;
      list[2 + 2 * copies] = v;
    }
    ++copies;
    __syncthreads();
  }
  for (int i = lane; i < MK; i += kLruThreads) {
    const int e = idx[i];
    slot_idx[i] = (e < 0 || e >= E || where[e] < 0) ? S : where[e];
  }
  for (int s = lane; s < S; s += kLruThreads) {
    slot_expert[s] = s_exp[s];
    slot_stamp[s] = s_stamp[s];
  }
  if (lane == 0) {
    slot_stamp[S] = now;
    list[0] = copies;
    if (n_copied) *n_copied = copies;
  }
}

// One block per (copy, part): the block copies its part of every segment of
// the expert (codes, scales, biases of gate, up and down).  Blocks past the
// call's copy count return at once (the grid is sized for M*K copies).
__global__ __launch_bounds__(kCopyThreads) void k_slot_copy(const StreamCopy P,
                                                            const int32_t* __restrict__ list) {
  const int c = blockIdx.x / P.parts, part = blockIdx.x - c * P.parts;
  if (c >= list[0]) return;
  const int e = list[1 + 2 * c], v = list[2 + 2 * c];
  const int tid = threadIdx.x;
  for (int g = 0; g < P.nseg; ++g) {
    const uint64_t bytes = P.bytes[g];
    const char* src = P.src[g] + (uint64_t)e * bytes;
    char* dst = P.dst[g] + (uint64_t)v * bytes;
    if ((bytes & 15) == 0) {
      const uint64_t units = bytes / 16;
      const uint64_t lo = units * part / P.parts, hi = units * (part + 1) / P.parts;
      const uint4* s4 = reinterpret_cast<const uint4*>(src);
      uint4* d4 = reinterpret_cast<uint4*>(dst);
      uint64_t i = lo + tid;
      for (; i + (uint64_t)kCopyThreads * (kCopyUnroll - 1) < hi; i += (uint64_t)kCopyThreads * kCopyUnroll) {
        uint4 r[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) r[u] = s4[i + (uint64_t)kCopyThreads * u];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) d4[i + (uint64_t)kCopyThreads * u] = r[u];
      }
      for (; i < hi; i += kCopyThreads) d4[i] = s4[i];
    } else {
      // a segment whose per-expert size is not a multiple of 16 bytes: bytes
      const uint64_t lo = bytes * part / P.parts, hi = bytes * (part + 1) / P.parts;
      for (uint64_t i = lo + tid; i < hi; i += kCopyThreads) dst[i] = src[i];
    }
  }
}

}  // namespace

int launch_stream_experts(const StreamCopy& P, const int32_t* idx, int MK, int E, int S,
                          int32_t* slot_expert, int64_t* slot_stamp, int32_t* slot_idx,
                          int32_t* list, int32_t* n_copied, hipStream_t s) {
  if (E > kMaxStreamExperts || S > kMaxStreamSlots || MK > S || P.parts < 1) return -9;
  hipLaunchKernelGGL(k_slot_lru, dim3(1), dim3(kLruThreads), 0, s, idx, MK, E, S, slot_expert,
                     slot_stamp, slot_idx, list, n_copied);
  hipLaunchKernelGGL(k_slot_copy, dim3(MK * P.parts), dim3(kCopyThreads), 0, s, P,
                     static_cast<const int32_t*>(list));
  return 0;
}

}  // namespace moeq
