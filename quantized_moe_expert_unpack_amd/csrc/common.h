// Device-side helpers shared by the HIP kernels of libmoeq (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moeq {

constexpr int kWave = 64;
constexpr int kGroup = 64;  // input columns per scale/bias group

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

}  // namespace moeq
