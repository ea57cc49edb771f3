// Device-side helpers shared by the HIP kernels of libmoeq (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moeq {

constexpr int kWave = 64;

// index of the group holding column c for a power-of-two group size gs (32,
// 64 or 128: validated on the host), without an integer division
__device__ __forceinline__ int group_of(int c, int gs) { return c >> __builtin_ctz((unsigned)gs); }

// n rounded up to a multiple of 4 (floats: to 16 bytes), for LDS regions
// followed by 16-byte stores
__host__ __device__ constexpr int pad4(int n) { return (n + 3) & ~3; }

// bf16 bit pattern -> fp32 (exact: bf16 is the top half of an fp32)
__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Code j (0-based) of a 16-byte chunk holding 128/BITS codes, low bits first.
template <int BITS>
__device__ __forceinline__ uint32_t chunk_code(const uint4& v, int j) {
  constexpr int kPer = 32 / BITS;
  constexpr uint32_t kMask = (1u << BITS) - 1u;
  const int w = j / kPer;
  const uint32_t word = w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
  return (word >> (BITS * (j % kPer))) & kMask;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// ---- arrival counting ------------------------------------------------------
// Device-scope atomics on one address serialize across the chip (about 11 ns
// each, measured on MI355X), so many arrivals are spread over kFan counters on
// separate 128-byte lines; whoever completes a sub-counter counts once in a top
// counter.  arrive() returns true for exactly one caller: the one completing
// all `total` arrivals.  Every counter is reset by the caller that completes
// it (no later arrival can touch it within the same launch), so the lines are
// zero again when the launch ends.
constexpr int kLineInts = 32;   // ints per 128-byte line
constexpr int kFan = 16;

// lines: (1 + kFan) * kLineInts ints: [0] top counter, [1 + s] sub-counter s
__device__ __forceinline__ bool arrive(int* lines, int slot, int total) {
  const int sub = slot % kFan;
  const int n_sub = total / kFan + (sub < total % kFan ? 1 : 0);
  int* c = lines + (1 + sub) * kLineInts;
  if (__hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != n_sub - 1)
    return false;
  __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int n_top = total < kFan ? total : kFan;
  if (__hip_atomic_fetch_add(lines, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != n_top - 1)
    return false;
  __hip_atomic_store(lines, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

}  // namespace moeq
