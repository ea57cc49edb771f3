// Routing selection on the device: softmax over all E experts, top-K by
// (score descending, index ascending), weights p[idx]/sum p[idx] (renorm) or
// p[idx].  markbaseengine MOE_ROUTER_WORKS_BREAKTHROUGH "Forward Pass
// Sequence" steps 1-4 and the flash-moe pipeline's "softmax + topK routing".
//
// Selection works on unique 64-bit keys: the fp64 logit's order-preserving bit
// pattern with its 10 lowest fraction bits replaced by (1023 - expert), so one
// integer compare orders by value and breaks ties towards the lower index
// (logits closer than 2^-42 relative compare as a tie; fp32 logits widened to
// fp64 have those bits zero and are ordered exactly).  Each wave of the block
// ranks its share of the keys, keeps every key whose rank in that share is
// < K (at most waves*K candidates), then the candidates are ranked.  The
// softmax itself is evaluated in fp64 on the exact logits.
#pragma once

#include "common.h"

namespace moeq {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;

// 64-bit maximum across the wave, left in every lane (DPP mirrors within
// rows of 16, permlane swaps across them; the maximum is indifferent to the
// mirrors' lane order)
template <int M>
__device__ __forceinline__ uint64_t xmax_u64(uint64_t v) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  if constexpr (M >= 16) {
    const auto rl = M == 32 ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                            : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto rh = M == 32 ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                            : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const uint64_t a = ((uint64_t)rh[0] << 32) | rl[0];
    const uint64_t b = ((uint64_t)rh[1] << 32) | rl[1];
    return a > b ? a : b;
  } else {
    constexpr int ctrl = M == 1 ? 0xB1 : M == 2 ? 0x4E : M == 4 ? 0x141 : 0x140;
    lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)lo, ctrl, 0xF, 0xF, false);
    hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)hi, ctrl, 0xF, 0xF, false);
    const uint64_t w = ((uint64_t)hi << 32) | lo;
    return v > w ? v : w;
  }
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = xmax_u64<32>(v);
  v = xmax_u64<16>(v);
  v = xmax_u64<8>(v);
  v = xmax_u64<4>(v);
  v = xmax_u64<2>(v);
  return xmax_u64<1>(v);
}

__device__ __forceinline__ uint64_t route_key(double v, int e) {
  uint64_t u = (uint64_t)__double_as_longlong(v);
  u = (u >> 63) ? ~u : (u | 0x8000000000000000ull);
  return (u & ~0x3FFull) | (uint64_t)(1023 - e);
}

// keys/vals (LDS) of one token -> K indices and weights.  Called by all NT
// threads of the block.
template <int NT>
__device__ void block_topk(const uint64_t* keys, const double* vals, int E, int K, int renorm,
                           int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  constexpr int kW = NT / kWave;
  __shared__ uint64_t cand[kW * kMaxTopK];
  __shared__ int ncand;
  __shared__ int sel[kMaxTopK];
  __shared__ double red[kW];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  if (tid == 0) ncand = 0;
  __syncthreads();
  const int q = (E + kW - 1) / kW;
  const int lo = min(E, wid * q), hi = min(E, lo + q);
  for (int a = lo + lane; a < hi; a += kWave) {
    const uint64_t ka = keys[a];
    int rank = 0;
#pragma unroll 8
    for (int j = lo; j < hi; ++j) rank += keys[j] > ka;
    if (rank < K) cand[atomicAdd(&ncand, 1)] = ka;
  }
  __syncthreads();
  const int nc = ncand;
  if (tid < nc) {
    const uint64_t kt = cand[tid];
    int rank = 0;
#pragma unroll 8
    for (int j = 0; j < nc; ++j) rank += cand[j] > kt;
    if (rank < K) sel[rank] = 1023 - (int)(kt & 0x3FFull);
  }
  __syncthreads();
  const double mx = vals[sel[0]];
  double total = 0.0;
  if (!renorm) {
    double part = 0.0;
    for (int e = tid; e < E; e += NT) part += exp(vals[e] - mx);
    part = wave_sum(part);
    if (lane == 0) red[wid] = part;
    __syncthreads();
    for (int w = 0; w < kW; ++w) total += red[w];
  } else {
    for (int k = 0; k < K; ++k) total += exp(vals[sel[k]] - mx);   // slot order
  }
  if (tid < K) {
    const int e = sel[tid];
    const float w = (float)(exp(vals[e] - mx) / total);
    idx_out[tid] = e;
    w_out[tid] = w;
  }
  __syncthreads();
}

}  // namespace moeq
