// Unpack/dequantize, the generic quantized matvec, and routing (router
// projection in fp64 + softmax/top-K) for libmoeq.
//
// Weight format: codes of BITS bits packed low-bits-first into uint32 words
// along the input dimension, one bf16 scale and bias per 64 input columns,
// w = scale*code + bias (flash-moe-inference skill page, matvec_4bit_fma;
// danveloper/flash-moe issue thread, per-tensor bit widths).  Rows are
// streamed in 16-byte chunks: a chunk holds 128/BITS codes and never straddles
// a group because a group is 8*BITS bytes (a multiple of 16).
#include "common.h"
#include "launch.h"

namespace moeq {

// ---------------------------------------------------------------------------
// qdequant: one thread per packed word
// ---------------------------------------------------------------------------
template <int BITS>
__global__ void __launch_bounds__(256) k_qdequant(const uint32_t* __restrict__ q,
                                                  const uint16_t* __restrict__ sc,
                                                  const uint16_t* __restrict__ bi, int64_t words,
                                                  int wpr, int cols, uint8_t* __restrict__ codes,
                                                  float* __restrict__ deq) {
  constexpr int kPer = 32 / BITS;
  constexpr uint32_t kMask = (1u << BITS) - 1u;
  const int groups = cols / kGroup;
  for (int64_t w = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; w < words;
       w += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = w / wpr;
    const int c0 = (int)(w - row * wpr) * kPer;
    const int64_t gidx = row * groups + c0 / kGroup;
    const float s = bf16_to_f32(sc[gidx]);
    const float b = bf16_to_f32(bi[gidx]);
    const uint32_t word = q[w];
    const int64_t o = row * cols + c0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t code = (word >> (BITS * j)) & kMask;
      if (codes) codes[o + j] = (uint8_t)code;
      if (deq) deq[o + j] = fmaf(s, (float)code, b);  // s*code is exact: one rounding
    }
  }
}

// ---------------------------------------------------------------------------
// qmatvec: one wave per output row, up to 4 tokens per pass over the row.
// fp32 dequantized weight (exactly the fp32 value of scale*code+bias), fp32
// accumulation, wave-shuffle reduction.
// ---------------------------------------------------------------------------
template <int BITS>
__global__ void __launch_bounds__(256) k_qmatvec(const uint32_t* __restrict__ q,
                                                 const uint16_t* __restrict__ sc,
                                                 const uint16_t* __restrict__ bi, int rows, int cols,
                                                 const float* __restrict__ x, int M,
                                                 float* __restrict__ y) {
  constexpr int kCpc = 128 / BITS;  // codes per 16-byte chunk
  const int lane = threadIdx.x & (kWave - 1);
  const int r = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (r >= rows) return;
  const int chunks = cols / kCpc;
  const int groups = cols / kGroup;
  const uint4* rq = reinterpret_cast<const uint4*>(q + (size_t)r * (cols / (32 / BITS)));
  const uint16_t* rs = sc + (size_t)r * groups;
  const uint16_t* rb = bi + (size_t)r * groups;
  for (int m0 = 0; m0 < M; m0 += 4) {
    const int mn = min(4, M - m0);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c = lane; c < chunks; c += kWave) {
      const uint4 v = rq[c];
      const int g = (c * kCpc) / kGroup;
      const float s = bf16_to_f32(rs[g]);
      const float b = bf16_to_f32(rb[g]);
      const float* xc = x + (size_t)m0 * cols + (size_t)c * kCpc;
#pragma unroll
      for (int j = 0; j < kCpc; j += 4) {
        float w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = fmaf(s, (float)chunk_code<BITS>(v, j + u), b);
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
          if (mm < mn) {
            const float4 xv = *reinterpret_cast<const float4*>(xc + (size_t)mm * cols + j);
            acc[mm] = fmaf(w[0], xv.x, acc[mm]);
            acc[mm] = fmaf(w[1], xv.y, acc[mm]);
            acc[mm] = fmaf(w[2], xv.z, acc[mm]);
            acc[mm] = fmaf(w[3], xv.w, acc[mm]);
          }
        }
      }
    }
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      const float t = wave_sum(acc[mm]);
      if (lane == 0 && mm < mn) y[(size_t)(m0 + mm) * rows + r] = t;
    }
  }
}

// ---------------------------------------------------------------------------
// Router projection in fp64: logits[m][e] = sum_k w_e,k * x_m,k with the fp32
// dequantized weight widened exactly and fp64 products/accumulation, so the
// top-K decision is taken on fp64 values.
// ---------------------------------------------------------------------------
template <int BITS>
__global__ void __launch_bounds__(256) k_router_f64(const uint32_t* __restrict__ q,
                                                    const uint16_t* __restrict__ sc,
                                                    const uint16_t* __restrict__ bi, int rows,
                                                    int cols, const float* __restrict__ x, int M,
                                                    double* __restrict__ logits,
                                                    float* __restrict__ logits32) {
  constexpr int kCpc = 128 / BITS;
  const int lane = threadIdx.x & (kWave - 1);
  const int r = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (r >= rows) return;
  const int chunks = cols / kCpc;
  const int groups = cols / kGroup;
  const uint4* rq = reinterpret_cast<const uint4*>(q + (size_t)r * (cols / (32 / BITS)));
  const uint16_t* rs = sc + (size_t)r * groups;
  const uint16_t* rb = bi + (size_t)r * groups;
  for (int m0 = 0; m0 < M; m0 += 2) {
    const int mn = min(2, M - m0);
    double acc[2] = {0.0, 0.0};
    for (int c = lane; c < chunks; c += kWave) {
      const uint4 v = rq[c];
      const int g = (c * kCpc) / kGroup;
      const float s = bf16_to_f32(rs[g]);
      const float b = bf16_to_f32(rb[g]);
      const float* xc = x + (size_t)m0 * cols + (size_t)c * kCpc;
#pragma unroll
      for (int j = 0; j < kCpc; j += 4) {
        double w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = (double)fmaf(s, (float)chunk_code<BITS>(v, j + u), b);
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          if (mm < mn) {
            const float4 xv = *reinterpret_cast<const float4*>(xc + (size_t)mm * cols + j);
            acc[mm] = fma(w[0], (double)xv.x, acc[mm]);
            acc[mm] = fma(w[1], (double)xv.y, acc[mm]);
            acc[mm] = fma(w[2], (double)xv.z, acc[mm]);
            acc[mm] = fma(w[3], (double)xv.w, acc[mm]);
          }
        }
      }
    }
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const double t = wave_sum(acc[mm]);
      if (lane == 0 && mm < mn) {
        logits[(size_t)(m0 + mm) * rows + r] = t;
        if (logits32) logits32[(size_t)(m0 + mm) * rows + r] = (float)t;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Softmax + explicit top-K, one wave per token.  K rounds of "largest
// remaining logit, lowest index on ties"; weights exp(l_k - max) over the sum
// of the chosen ones (renorm) or over all E (softmax values).  fp64 math.
// ---------------------------------------------------------------------------
constexpr int kMaxPerLane = 16;  // E <= 1024

__device__ __forceinline__ bool better(double v, int i, double ov, int oi) {
  return v > ov || (v == ov && i < oi);
}

__global__ void __launch_bounds__(256) k_topk(const double* __restrict__ l64,
                                              const float* __restrict__ l32, int M, int E, int K,
                                              int renorm, int32_t* __restrict__ idx,
                                              float* __restrict__ wout) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (t >= M) return;
  double v[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + kWave * i;
    double val = -INFINITY;
    if (e < E) val = l64 ? l64[(size_t)t * E + e] : (double)l32[(size_t)t * E + e];
    v[i] = val;
  }
  double mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) mx = fmax(mx, v[i]);
  mx = wave_max(mx);
  double total = 0.0;
  if (!renorm) {
    double part = 0.0;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i)
      if (lane + kWave * i < E) part += exp(v[i] - mx);
    total = wave_sum(part);
  }
  double selv[16];
  int seli[16];
  double selsum = 0.0;
  for (int k = 0; k < K; ++k) {
    double bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + kWave * i;
      if (e < E && better(v[i], e, bv, bi)) { bv = v[i]; bi = e; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i)
      if (lane + kWave * i == bi) v[i] = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
      if (kk == k) { selv[kk] = bv; seli[kk] = bi; }
    selsum += exp(bv - mx);
  }
  if (renorm) total = selsum;
  if (lane < K) {
    double sv = 0.0;
    int si = 0;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
      if (kk == lane) { sv = selv[kk]; si = seli[kk]; }
    idx[(size_t)t * K + lane] = si;
    wout[(size_t)t * K + lane] = (float)(exp(sv - mx) / total);
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
#define MOEQ_BITS_LAUNCH(bits, KERNEL, GRID, ...)                                          \
  do {                                                                                    \
    if ((bits) == 8) hipLaunchKernelGGL(KERNEL<8>, GRID, dim3(256), 0, __VA_ARGS__);       \
    else if ((bits) == 4) hipLaunchKernelGGL(KERNEL<4>, GRID, dim3(256), 0, __VA_ARGS__);  \
    else hipLaunchKernelGGL(KERNEL<2>, GRID, dim3(256), 0, __VA_ARGS__);                   \
  } while (0)

int launch_qdequant(const QT& W, uint8_t* codes, float* deq, hipStream_t s) {
  const int wpr = W.cols * W.bits / 32;
  const int64_t words = (int64_t)W.batch * W.rows * wpr;
  if (words == 0) return 0;
  const int64_t want = (words + 255) / 256;
  const int blocks = (int)(want < 65536 ? want : 65536);
  MOEQ_BITS_LAUNCH(W.bits, k_qdequant, dim3(blocks), s, W.q, W.scales, W.biases, words, wpr,
                   W.cols, codes, deq);
  return 0;
}

int launch_qmatvec(const QT& W, const float* x, int M, float* y, hipStream_t s) {
  const int blocks = (W.rows + 3) / 4;
  MOEQ_BITS_LAUNCH(W.bits, k_qmatvec, dim3(blocks), s, W.q, W.scales, W.biases, W.rows, W.cols, x,
                   M, y);
  return 0;
}

int launch_router_f64(const QT& W, const float* x, int M, double* logits, float* logits32,
                      hipStream_t s) {
  const int blocks = (W.rows + 3) / 4;
  MOEQ_BITS_LAUNCH(W.bits, k_router_f64, dim3(blocks), s, W.q, W.scales, W.biases, W.rows, W.cols,
                   x, M, logits, logits32);
  return 0;
}

int launch_topk(const double* l64, const float* l32, int M, int E, int K, int renorm, int32_t* idx,
                float* w, hipStream_t s) {
  const int blocks = (M + 3) / 4;
  hipLaunchKernelGGL(k_topk, dim3(blocks), dim3(256), 0, s, l64, l32, M, E, K, renorm, idx, w);
  return 0;
}

}  // namespace moeq
