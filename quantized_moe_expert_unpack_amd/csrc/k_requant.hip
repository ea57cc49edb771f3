// 2-bit requantization of a 4- or 8-bit affine tensor, group by group
// (flash-moe-inference skill page: the 4-bit to 2-bit conversion step of the
// setup and repack_experts_2bit.py in the repository layout; the page gives no
// arithmetic).  For one group with scale s, bias b and codes q the weights are
// w = s*q + b; the 2-bit grid spans the group's exact minimum lo to maximum hi
// in three equal steps, every weight takes the nearest grid point (ties to the
// even code), a group without spread takes code 0, and the stored scale and
// bias are (hi - lo)/3 and lo rounded once to bf16.
//
// HBM-bound and elementwise.  A lane takes one 16-byte chunk of codes (32 at
// 4 bits, 16 at 8 bits); the 2, 4 or 8 lanes of one group (consecutive lanes,
// since chunks run along the rows and a group never crosses a row) reduce the
// group's smallest and largest code with lane shuffles.  Everything after
// that is integer work on the codes: for s > 0 the weight's position on the
// grid is 3*(q - qmin)/span with span = qmax - qmin (for s < 0 the same with
// the codes reflected), so the rounded code is a count of three integer
// thresholds, applied to four codes at a time within a word.  Only the two
// stored values are floating point; each is formed as an fp32 value rounded
// to odd and then rounded to nearest-even bf16, which equals rounding the
// exact value once.
#include "common.h"
#include "launch.h"

namespace moeq {
namespace {

constexpr int kRqThreads = 256;
constexpr int kRqPer = 2;              // chunks per thread, kRqThreads apart

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// bf16 nearest to the exact value hi + err, where hi is that value rounded to
// nearest fp32 and err the exact remainder: round to odd in fp32 (truncate,
// then set the last bit when inexact), then to nearest-even bf16.  Round to
// odd with more than one extra bit makes the second rounding exact.
__device__ __forceinline__ uint32_t bf16_from_sum(float hi, float err) {
  uint32_t u = __float_as_uint(hi);
  if (err != 0.0f) {
    // the exact value lies beyond hi (same sign as hi) or between hi and the
    // float one step closer to zero
    const bool beyond = (err > 0.0f) == (hi > 0.0f);
    u = (beyond ? u : u - 1u) | 1u;
  }
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// q2 for the codes in the bytes (FB = 8) or 16-bit halves (FB = 16) of d: the
// count of thresholds d >= A_k, k = 1..3, each read as the top bit of the
// field d + (2^(FB-1) - A_k); k1..k3 hold 2^(FB-1) - A_k in every field, and
// no field carries into the next (d < 2^(FB-1), A_k >= 1).
template <int FB>   // field bits: 8 or 16
__device__ __forceinline__ uint32_t thresholds(uint32_t d, uint32_t k1, uint32_t k2, uint32_t k3) {
  constexpr uint32_t one = FB == 8 ? 0x01010101u : 0x00010001u;
  constexpr int top = FB - 1;
  return (((d + k1) >> top) & one) + (((d + k2) >> top) & one) + (((d + k3) >> top) & one);
}

template <int BITS>
__global__ __launch_bounds__(kRqThreads) void k_requant2(
    const u32x4* __restrict__ q, const uint16_t* __restrict__ sc, const uint16_t* __restrict__ bi,
    int nchunks, int lsh, uint32_t* __restrict__ q2, uint16_t* __restrict__ sc2,
    uint16_t* __restrict__ bi2) {
  constexpr uint32_t kMax = (1u << BITS) - 1u;
  constexpr int FB = BITS == 4 ? 8 : 16;           // field width of the threshold step
  constexpr uint32_t rep = FB == 8 ? 0x01010101u : 0x00010001u;
  constexpr uint32_t top = 1u << (FB - 1);
  const int lanes = 1 << lsh;                      // lanes per group
  u32x4 v[kRqPer];
  uint32_t sb[kRqPer];
  int c[kRqPer];
#pragma unroll
  for (int j = 0; j < kRqPer; ++j) {
    c[j] = (blockIdx.x * kRqPer + j) * kRqThreads + (int)threadIdx.x;
    const int cc = min(c[j], nchunks - 1);
    v[j] = q[cc];
    sb[j] = (uint32_t)sc[cc >> lsh] | ((uint32_t)bi[cc >> lsh] << 16);
  }
#pragma unroll
  for (int j = 0; j < kRqPer; ++j) {
    // the group's smallest and largest code
    uint32_t mn = kMax, mx = 0u;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
      for (int k = 0; k < 32 / BITS; ++k) {
        const uint32_t code = (v[j][w] >> (BITS * k)) & kMax;
        mn = min(mn, code);
        mx = max(mx, code);
      }
    }
    for (int m = 1; m < lanes; m <<= 1) {
      mn = min(mn, (uint32_t)__shfl_xor((int)mn, m));
      mx = max(mx, (uint32_t)__shfl_xor((int)mx, m));
    }
    const float s = bf16_to_f32(sb[j] & 0xFFFFu), b = bf16_to_f32(sb[j] >> 16);
    const int span = (int)(mx - mn);
    const bool neg = s < 0.0f;
    // the minimum weight sits at the smallest code (s > 0) or the largest
    const float xlo = __fmul_rn(s, (float)(neg ? mx : mn));      // exact: <= 16 significant bits
    const float lo = __fadd_rn(xlo, b);
    const float bb = __fsub_rn(lo, xlo);
    const float lo_err = __fadd_rn(__fsub_rn(xlo, __fsub_rn(lo, bb)), __fsub_rn(b, bb));
    const float xs = __fmul_rn(fabsf(s), (float)span);            // exact
    const float st = __fdiv_rn(xs, 3.0f);
    const float st_err = __fmaf_rn(-st, 3.0f, xs);               // exact remainder
    const uint32_t s2 = bf16_from_sum(st, st_err);
    const uint32_t b2 = bf16_from_sum(lo, lo_err);
    // position on the grid 3*d/span with d = distance from the minimum's
    // code: code k+1 from 6d > (2k+1)*span, the ties 6d == 3*span going up
    // to the even code 2 and the others down
    const bool flat = span == 0 || s == 0.0f;
    const int a1 = flat ? (int)top : span / 6 + 1;
    const int a2 = flat ? (int)top : (span + 1) / 2;
    const int a3 = flat ? (int)top : (5 * span) / 6 + 1;
    const uint32_t k1 = (top - (uint32_t)a1) * rep, k2 = (top - (uint32_t)a2) * rep,
                   k3 = (top - (uint32_t)a3) * rep;
    const uint32_t flip = neg ? 0xFFFFFFFFu : 0u;                // s < 0: reflect q -> kMax - q
    const uint32_t ref = (neg ? kMax - mx : mn) * rep;
    uint32_t out[BITS == 4 ? 2 : 1] = {};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x = v[j][w] ^ flip;
      if constexpr (BITS == 4) {
        // even codes (0,2,4,6) in the low nibbles, odd ones in the high
        const uint32_t ev = thresholds<8>((x & 0x0F0F0F0Fu) - ref, k1, k2, k3);
        const uint32_t od = thresholds<8>(((x >> 4) & 0x0F0F0F0Fu) - ref, k1, k2, k3);
        const uint32_t z = ev | (od << 2);           // byte i: codes 2i, 2i+1 (4 bits)
        const uint32_t y = z | (z >> 4);             // bytes 0 and 2: codes 0-3 and 4-7
        const uint32_t h = (y & 0xFFu) | ((y >> 8) & 0xFF00u);
        out[w >> 1] |= h << (16 * (w & 1));
      } else {
        const uint32_t ev = thresholds<16>((x & 0x00FF00FFu) - ref, k1, k2, k3);
        const uint32_t od = thresholds<16>(((x >> 8) & 0x00FF00FFu) - ref, k1, k2, k3);
        const uint32_t z = ev | (od << 2);           // half i: codes 2i, 2i+1
        out[0] |= ((z & 0xFu) | ((z >> 12) & 0xF0u)) << (8 * w);
      }
    }
    if (c[j] < nchunks) {
      if constexpr (BITS == 4)
        reinterpret_cast<uint2*>(q2)[c[j]] = make_uint2(out[0], out[1]);
      else
        q2[c[j]] = out[0];
      if ((c[j] & (lanes - 1)) == 0) {
        sc2[c[j] >> lsh] = (uint16_t)s2;
        bi2[c[j] >> lsh] = (uint16_t)b2;
      }
    }
  }
}

}  // namespace

// The source's chunks run back to back over every row of every matrix, and
// a group of gs columns is gs / (128 / bits) consecutive chunks.
int launch_requant_2bit(const QT& W, uint32_t* q2, uint16_t* s2, uint16_t* b2, hipStream_t st) {
  const size_t codes = (size_t)W.batch * W.rows * W.cols;
  const int cpc = 128 / W.bits;
  const int nchunks = (int)(codes / cpc);
  const int lsh = __builtin_ctz((unsigned)(W.group_size / cpc));
  const int per_block = kRqThreads * kRqPer;
  const dim3 grid((nchunks + per_block - 1) / per_block);
  const u32x4* q = reinterpret_cast<const u32x4*>(W.q);
  if (W.bits == 4)
    k_requant2<4><<<grid, kRqThreads, 0, st>>>(q, W.scales, W.biases, nchunks, lsh, q2, s2, b2);
  else
    k_requant2<8><<<grid, kRqThreads, 0, st>>>(q, W.scales, W.biases, nchunks, lsh, q2, s2, b2);
  return 0;
}

}  // namespace moeq
