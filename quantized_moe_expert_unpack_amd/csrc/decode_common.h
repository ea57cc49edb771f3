// Device helpers shared by the decode kernels (one-launch layer and batched
// decode): chunked dequantizing dot products over LDS-resident activations and
// VALU-only wave reductions.
#pragma once

#include "common.h"

namespace moeq {

// Activations live in LDS chunk-interleaved: float4 number f of chunk c sits at
// a4[f * stride + c], so lanes working on consecutive chunks read consecutive
// 16-byte words (a plain [c][f] layout puts them 16*BITS bytes apart and every
// read becomes a many-way bank conflict).
//
// dot of one 16-byte chunk of BITS-bit codes with its activations
// A word of 2- or 4-bit codes is converted in byte passes: pass m of the
// word has code 4b + m (2-bit) or 2b + m (4-bit) in byte b, and each byte
// becomes a float with one byte-to-float instruction (the empty asm keeps
// the compiler from turning the mask back into one bit-field extract per
// code); 8-bit words are their own single pass.
template <int BITS>
__device__ __forceinline__ uint32_t code_pass(uint32_t w, int m) {
  uint32_t t = w;
  if constexpr (BITS == 2) t = (w >> (2 * m)) & 0x03030303u;
  else if constexpr (BITS == 4) t = (w >> (4 * m)) & 0x0F0F0F0Fu;
  asm volatile("" : "+v"(t));
  return t;
}

__device__ __forceinline__ float f4c(const float4& v, int c) {
  return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}

template <int BITS>
__device__ __forceinline__ float chunk_dot(const uint4& v, const float4* a4, int stride) {
  constexpr int kF = 8 / BITS;                 // float4s of activations per word
  constexpr int kPasses = 8 / BITS;
  float d = 0.f;
#pragma unroll
  for (int wi = 0; wi < 4; ++wi) {
    const uint32_t w = wi == 0 ? v.x : wi == 1 ? v.y : wi == 2 ? v.z : v.w;
    float4 av[kF];
#pragma unroll
    for (int f = 0; f < kF; ++f) av[f] = a4[(wi * kF + f) * stride];
#pragma unroll
    for (int m = 0; m < kPasses; ++m) {
      const uint32_t t = code_pass<BITS>(w, m);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int j = BITS == 2 ? 4 * b + m : BITS == 4 ? 2 * b + m : b;   // code within the word
        d = fmaf((float)((t >> (8 * b)) & 0xFFu), f4c(av[j / 4], j % 4), d);
      }
    }
  }
  return d;
}

// position (in float4 units) of float4 number i of a vector cut into chunks of
// CPC floats, nch chunks, in the interleaved layout
template <int CPC>
__device__ __forceinline__ int ilv(int i, int nch) {
  constexpr int kF = CPC / 4;
  return (i % kF) * nch + i / kF;
}

// chunk sums of an interleaved activation vector (nch chunks of CPC floats)
template <int CPC>
__device__ __forceinline__ void chunk_sums(const float4* a4, float* sums, int nch) {
  for (int c = threadIdx.x; c < nch; c += blockDim.x) {
    float s = 0.f;
#pragma unroll
    for (int f = 0; f < CPC / 4; ++f) {
      const float4 v = a4[f * nch + c];
      s += (v.x + v.y) + (v.z + v.w);
    }
    sums[c] = s;
  }
}

// ---- transposed wave reductions -------------------------------------------
// A wave holds N per-lane partial sums (N rows); an exchange step across lane
// bit M halves the live values per lane: a lane with bit M clear keeps the
// first half of the rows, a lane with bit M set the second half, each adding
// its partner's matching partial.  After log2(N) such steps every lane holds a
// single row's partial, which the remaining steps reduce normally; N rows
// cost about N + 6 exchanges instead of 6N.  Exchanges are VALU-only: DPP
// quad permutes and row (half) mirrors inside 16-lane rows, and gfx950's
// v_permlane16/32_swap across rows.  A mirror also flips the lower lane bits,
// which keeps every reduction tree exact because later steps never look at
// the bits above M again.
template <int M>
__device__ __forceinline__ float xdpp(float v) {
  constexpr int ctrl = M == 1 ? 0xB1 : M == 2 ? 0x4E : M == 4 ? 0x141 : 0x140;
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xF, 0xF, false));
}

// pair (x, y) -> x summed over the pair for lanes with bit M clear, y for set
template <int M>
__device__ __forceinline__ float tpair(float x, float y, int lane) {
  if constexpr (M == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    const bool hi = lane & M;
    return (hi ? y : x) + xdpp<M>(hi ? x : y);
  }
}

// plain step: v summed with its partner across bit M
template <int M>
__device__ __forceinline__ float tplain(float v) {
  if constexpr (M >= 16) return tpair<M>(v, v, 0);
  else return v + xdpp<M>(v);
}

// N values, transposed steps over masks TOP, TOP/2, ... (log2 N of them),
// then plain steps down to mask 1.  Returns the lane's single value.
template <int N, int TOP>
__device__ __forceinline__ float treduce(float* v, int lane) {
  if constexpr (N > 1) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) v[i] = tpair<TOP>(v[i], v[i + N / 2], lane);
    return treduce<N / 2, TOP / 2>(v, lane);
  } else if constexpr (TOP >= 1) {
    v[0] = tplain<TOP>(v[0]);
    return treduce<1, TOP / 2>(v, lane);
  } else {
    return v[0];
  }
}

// the row (value index) a lane holds after treduce<N, TOP>: bits TOP, TOP/2, ...
template <int N, int TOP>
__device__ __forceinline__ int tindex(int lane) {
  int r = 0;
#pragma unroll
  for (int b = TOP, w = N / 2; w >= 1; b >>= 1, w >>= 1) r += (lane & b) ? w : 0;
  return r;
}

}  // namespace moeq
