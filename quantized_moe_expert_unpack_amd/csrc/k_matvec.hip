// Unpack/dequantize, the generic quantized matvec, and routing (router
// projection in fp64 + softmax/top-K) for libmoeq.
//
// Weight format: codes of BITS bits packed low-bits-first into uint32 words
// along the input dimension, one bf16 scale and bias per group of gs input
// columns (gs = 32, 64 or 128; 64 or 128 at 2 bits), w = scale*code + bias
// (flash-moe-inference skill page, matvec_4bit_fma; danveloper/flash-moe issue
// thread, per-tensor bit widths; ml-explore/mlx issue #3856, the repros at
// group_size 32).  Rows are streamed in 16-byte chunks: a chunk holds 128/BITS
// codes and never straddles a group because gs is a multiple of 128/BITS.
#include "common.h"
#include "launch.h"
#include "topk.h"

namespace moeq {

// ---------------------------------------------------------------------------
// qdequant: one thread per packed word
// ---------------------------------------------------------------------------
template <int BITS>
__global__ void __launch_bounds__(256) k_qdequant(const uint32_t* __restrict__ q,
                                                  const uint16_t* __restrict__ sc,
                                                  const uint16_t* __restrict__ bi, int64_t words,
                                                  int wpr, int cols, int gs, uint8_t* __restrict__ codes,
                                                  float* __restrict__ deq) {
  constexpr int kPer = 32 / BITS;
  constexpr uint32_t kMask = (1u << BITS) - 1u;
  const int groups = cols / gs;
  for (int64_t w = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; w < words;
       w += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = w / wpr;
    const int c0 = (int)(w - row * wpr) * kPer;
    const int64_t gidx = row * groups + group_of(c0, gs);
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
                                                 int gs, const float* __restrict__ x, int M,
                                                 float* __restrict__ y) {
  constexpr int kCpc = 128 / BITS;  // codes per 16-byte chunk
  const int lane = threadIdx.x & (kWave - 1);
  const int r = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (r >= rows) return;
  const int chunks = cols / kCpc;
  const int groups = cols / gs;
  const uint4* rq = reinterpret_cast<const uint4*>(q + (size_t)r * (cols / (32 / BITS)));
  const uint16_t* rs = sc + (size_t)r * groups;
  const uint16_t* rb = bi + (size_t)r * groups;
  for (int m0 = 0; m0 < M; m0 += 4) {
    const int mn = min(4, M - m0);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c = lane; c < chunks; c += kWave) {
      const uint4 v = rq[c];
      const int g = group_of(c * kCpc, gs);
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
// mxfp4 (E2M1 codes, one E8M0 scale byte per 32 columns, no bias)
// ---------------------------------------------------------------------------
// E2M1: bit 3 the sign, bits 2-1 the exponent (bias 1), bit 0 the mantissa
__device__ __forceinline__ float e2m1(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const float mag = e == 0 ? 0.5f * (float)m : (1.0f + 0.5f * (float)m) * (float)(1u << (e - 1));
  return (c & 8u) ? -mag : mag;
}

// one thread per packed word: codes, and value * 2^(e - 127) (exact: a
// two-bit significand times a power of two, by ldexp, subnormals included)
__global__ void __launch_bounds__(256) k_qdequant_mx(const uint32_t* __restrict__ q,
                                                     const uint8_t* __restrict__ sc, int64_t words,
                                                     int wpr, int cols, uint8_t* __restrict__ codes,
                                                     float* __restrict__ deq) {
  const int groups = cols / 32;
  for (int64_t w = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; w < words;
       w += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = w / wpr;
    const int c0 = (int)(w - row * wpr) * 8;
    const int e = (int)sc[row * groups + c0 / 32] - 127;
    const uint32_t word = q[w];
    const int64_t o = row * cols + c0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t code = (word >> (4 * j)) & 15u;
      if (codes) codes[o + j] = (uint8_t)code;
      if (deq) deq[o + j] = ldexpf(e2m1(code), e);
    }
  }
}

// one wave per output row, up to 4 tokens per pass; a 16-byte chunk is one
// group of 32: the chunk's dot in fp32, then scaled by its power of two
__global__ void __launch_bounds__(256) k_qmatvec_mx(const uint32_t* __restrict__ q,
                                                    const uint8_t* __restrict__ sc, int rows,
                                                    int cols, const float* __restrict__ x, int M,
                                                    float* __restrict__ y) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (r >= rows) return;
  const int chunks = cols / 32;
  const uint4* rq = reinterpret_cast<const uint4*>(q + (size_t)r * (cols / 8));
  const uint8_t* rs = sc + (size_t)r * chunks;
  for (int m0 = 0; m0 < M; m0 += 4) {
    const int mn = min(4, M - m0);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c = lane; c < chunks; c += kWave) {
      const uint4 v = rq[c];
      const int e = (int)rs[c] - 127;
      const float* xc = x + (size_t)m0 * cols + (size_t)c * 32;
      float d[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 32; j += 4) {
        float w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = e2m1(chunk_code<4>(v, j + u));
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
          if (mm < mn) {
            const float4 xv = *reinterpret_cast<const float4*>(xc + (size_t)mm * cols + j);
            d[mm] = fmaf(w[0], xv.x, d[mm]);
            d[mm] = fmaf(w[1], xv.y, d[mm]);
            d[mm] = fmaf(w[2], xv.z, d[mm]);
            d[mm] = fmaf(w[3], xv.w, d[mm]);
          }
        }
      }
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) acc[mm] += ldexpf(d[mm], e);
    }
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      const float t = wave_sum(acc[mm]);
      if (lane == 0 && mm < mn) y[(size_t)(m0 + mm) * rows + r] = t;
    }
  }
}

// ---------------------------------------------------------------------------
// Routing (selection in topk.h)
// ---------------------------------------------------------------------------
constexpr int kRouteThreads = 256;
constexpr int kMaxE = kMaxExperts;
constexpr int kLastTopkMaxM = 4;   // tokens of the one-launch router form (k_router)

// splits of the hidden dimension for k_router_mma: enough blocks to fill
// the chip (16 tokens x 64 rows per block), at most 8
constexpr int kMaxParts = 8;
int router_splits(int M, int E) {
  const int blocks = ((M + 15) / 16) * ((E + 63) / 64);
  return blocks >= 512 ? 1 : (512 / blocks < kMaxParts ? 512 / blocks : kMaxParts);
}
constexpr int kMmaMinM = 16;   // the MFMA router from this many tokens


// Router projection in fp64 (the fp32 dequantized weight widened exactly,
// fp64 products and sums), one wave per router row and token.  With
// LAST_TOPK the block that finishes last (arrival counter) runs top-K for all
// M tokens and resets the counter; otherwise logits stay in the workspace for
// k_topk_wave.
template <int BITS, bool LAST_TOPK>
__global__ void __launch_bounds__(kRouteThreads) k_router(QT W, const float* __restrict__ x, int M,
                                                          int K, int renorm,
                                                          double* __restrict__ logits,
                                                          int* __restrict__ ctr,
                                                          float* __restrict__ logits32,
                                                          int32_t* __restrict__ idx,
                                                          float* __restrict__ wout) {
  __shared__ uint64_t keys[kMaxE];
  __shared__ double vals[kMaxE];
  __shared__ int s_last;
  constexpr int kCpc = 128 / BITS;
  const int rows = W.rows, cols = W.cols;
  const int lane = threadIdx.x & (kWave - 1);
  const int r = blockIdx.x * (kRouteThreads / kWave) + (threadIdx.x / kWave);
  if (r < rows) {
    const int chunks = cols / kCpc;
    const int groups = cols / W.group_size;
    const uint4* rq = reinterpret_cast<const uint4*>(W.q + (size_t)r * (cols / (32 / BITS)));
    const uint16_t* rs = W.scales + (size_t)r * groups;
    const uint16_t* rb = W.biases + (size_t)r * groups;
    // per lane its chunks lane, lane + 64, ... in order, one fp64 chain per
    // token (M <= 4); four chunks' loads go out together, and a weight is
    // dequantized once for all tokens
    constexpr int kB = 4;
    double acc[kLastTopkMaxM];
#pragma unroll
    for (int m = 0; m < kLastTopkMaxM; ++m) acc[m] = 0.0;
    for (int c0 = lane; c0 < chunks; c0 += kB * kWave) {
      uint4 v[kB];
      float s[kB], b[kB];
#pragma unroll
      for (int q = 0; q < kB; ++q) {
        const int c = min(c0 + q * kWave, chunks - 1);      // clamped: always a valid address
        const int g = group_of(c * kCpc, W.group_size);
        v[q] = rq[c];
        s[q] = bf16_to_f32(rs[g]);
        b[q] = bf16_to_f32(rb[g]);
      }
#pragma unroll
      for (int q = 0; q < kB; ++q) {
        const int c = c0 + q * kWave;
        if (c >= chunks) break;
#pragma unroll
        for (int j = 0; j < kCpc; j += 4) {
          double w[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = (double)fmaf(s[q], (float)chunk_code<BITS>(v[q], j + i), b[q]);
#pragma unroll
          for (int m = 0; m < kLastTopkMaxM; ++m) {
            if (m < M) {
              const float4 xv = *reinterpret_cast<const float4*>(x + (size_t)m * cols + (size_t)c * kCpc + j);
              acc[m] = fma(w[0], (double)xv.x, acc[m]);
              acc[m] = fma(w[1], (double)xv.y, acc[m]);
              acc[m] = fma(w[2], (double)xv.z, acc[m]);
              acc[m] = fma(w[3], (double)xv.w, acc[m]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < kLastTopkMaxM; ++m) {
      if (m < M) {
        const double a = wave_sum(acc[m]);
        if (lane == 0) {
          __hip_atomic_store(logits + (size_t)m * rows + r, a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (logits32) logits32[(size_t)m * rows + r] = (float)a;
        }
      }
    }
  }
  if (!LAST_TOPK) return;
  // logits went out with coherent (agent-scope) stores: drain, then announce
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) s_last = arrive(ctr, blockIdx.x, gridDim.x);
  __syncthreads();
  if (!s_last) return;
  for (int m = 0; m < M; ++m) {
    double v[kMaxE / kRouteThreads];               // all loads in flight first
#pragma unroll
    for (int j = 0; j < kMaxE / kRouteThreads; ++j) {
      const int e = threadIdx.x + kRouteThreads * j;
      v[j] = e < rows ? __hip_atomic_load(logits + (size_t)m * rows + e, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT)
                      : 0.0;
    }
#pragma unroll
    for (int j = 0; j < kMaxE / kRouteThreads; ++j) {
      const int e = threadIdx.x + kRouteThreads * j;
      if (e < rows) {
        vals[e] = v[j];
        keys[e] = route_key(v[j], e);
      }
    }
    __syncthreads();
    block_topk<kRouteThreads>(keys, vals, rows, K, renorm, idx + (size_t)m * K, wout + (size_t)m * K);
  }
}

// Router projection for many tokens, the same fp64 arithmetic as k_router:
// one wave per (router row, kRouteTM tokens).  Each weight is dequantized and
// widened once and feeds kRouteTM independent fp64 chains; the grid spans
// rows and token blocks so that it fills the chip.
constexpr int kRouteTM = 8;
template <int BITS>
__global__ void __launch_bounds__(kRouteThreads) k_router_many(QT W, const float* __restrict__ x,
                                                               int M, double* __restrict__ logits,
                                                               float* __restrict__ logits32) {
  constexpr int kCpc = 128 / BITS;
  const int rows = W.rows, cols = W.cols;
  const int lane = threadIdx.x & (kWave - 1);
  const int r = blockIdx.x * (kRouteThreads / kWave) + (threadIdx.x / kWave);
  const int m0 = blockIdx.y * kRouteTM;
  if (r >= rows) return;
  const int nm = min(kRouteTM, M - m0);
  const int chunks = cols / kCpc;
  const int groups = cols / W.group_size;
  const uint4* rq = reinterpret_cast<const uint4*>(W.q + (size_t)r * (cols / (32 / BITS)));
  const uint16_t* rs = W.scales + (size_t)r * groups;
  const uint16_t* rb = W.biases + (size_t)r * groups;
  double acc[kRouteTM];
#pragma unroll
  for (int t = 0; t < kRouteTM; ++t) acc[t] = 0.0;
  for (int c = lane; c < chunks; c += kWave) {
    const uint4 v = rq[c];
    const int g = group_of(c * kCpc, W.group_size);
    const float s = bf16_to_f32(rs[g]);
    const float b = bf16_to_f32(rb[g]);
#pragma unroll
    for (int j = 0; j < kCpc; j += 4) {
      float4 xv[kRouteTM];
#pragma unroll
      for (int t = 0; t < kRouteTM; ++t)   // rows past the last token re-read token 0's x
        xv[t] = *reinterpret_cast<const float4*>(x + (size_t)(m0 + (t < nm ? t : 0)) * cols +
                                                 (size_t)c * kCpc + j);
      double w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = (double)fmaf(s, (float)chunk_code<BITS>(v, j + q), b);
#pragma unroll
      for (int t = 0; t < kRouteTM; ++t) {
        acc[t] = fma(w[0], (double)xv[t].x, acc[t]);
        acc[t] = fma(w[1], (double)xv[t].y, acc[t]);
        acc[t] = fma(w[2], (double)xv[t].z, acc[t]);
        acc[t] = fma(w[3], (double)xv[t].w, acc[t]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int t = 0; t < kRouteTM; ++t) {
    const double a = wave_sum(acc[t]);
    if (lane == 0 && t < nm) {
      logits[(size_t)(m0 + t) * rows + r] = a;
      if (logits32) logits32[(size_t)(m0 + t) * rows + r] = (float)a;
    }
  }
}

// top-K for many tokens, one wave per token (four per block): the same
// unique keys and rank order as block_topk, the selection by K rounds of a
// wave-wide maximum, with the weights from the same fp64 expressions
// (renormalized: the K exponentials summed in slot order; otherwise the
// partial sums of 64 experts each, added in expert order).  PER keys per
// lane: E <= 64 * PER.
// With nparts > 1 the fp64 logits arrive as nparts partial sums (a split
// reduction dimension, part p at p * M * E) and are added here in part order;
// l32_out, if given, receives them rounded to fp32.
template <int PER>
__global__ void __launch_bounds__(kRouteThreads) k_topk_wave(const double* __restrict__ l64,
                                                             const float* __restrict__ l32, int M,
                                                             int E, int K, int renorm,
                                                             int32_t* __restrict__ idx,
                                                             float* __restrict__ wout, int nparts,
                                                             float* __restrict__ l32_out) {
  constexpr int kPer = PER;
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (kRouteThreads / kWave) + threadIdx.x / kWave;
  if (t >= M) return;                            // whole waves leave together
  const size_t row = (size_t)t * E;
  uint64_t key[kPer];
  double val[kPer];
  uint32_t live = 0u;                            // bit j: slot j holds an unselected key
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = lane + kWave * j;
    val[j] = 0.0;
    key[j] = 0ull;
    if (e < E) {
      if (l64) {
        // every part's load first (at most kMaxParts), then the sum in part order
        double pv[kMaxParts];
#pragma unroll
        for (int p = 0; p < kMaxParts; ++p)
          pv[p] = p < nparts ? l64[(size_t)p * M * E + row + e] : 0.0;
        double v = pv[0];
#pragma unroll
        for (int p = 1; p < kMaxParts; ++p)
          if (p < nparts) v += pv[p];
        val[j] = v;
        if (l32_out) l32_out[row + e] = (float)v;
      } else {
        val[j] = (double)l32[row + e];
      }
      key[j] = route_key(val[j], e);
      live |= 1u << j;
    }
  }
  int my_e = 0;                                  // lane k < K: the expert of slot k
  for (int k = 0; k < K; ++k) {
    uint64_t local = 0ull;
    int lj = -1;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (((live >> j) & 1u) && (lj < 0 || key[j] > local)) {
        local = key[j];
        lj = j;
      }
    const uint64_t best = wave_max_u64(local);
    if (lj >= 0 && local == best) live &= ~(1u << lj);   // keys are unique: one lane
    if (lane == k) my_e = 1023 - (int)(best & 0x3FFull);
  }
  // the selected experts' logits from the lanes holding them
  double v = 0.0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const double vj = __shfl(val[j], my_e & (kWave - 1), kWave);
    if ((my_e >> 6) == j) v = vj;
  }
  if (lane >= K) v = 0.0;
  const double mx = __shfl(v, 0, kWave);
  double total = 0.0;
  if (renorm) {
    const double ex = lane < K ? exp(v - mx) : 0.0;
    for (int k = 0; k < K; ++k) total += __shfl(ex, k, kWave);   // slot order
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (kWave * j >= E) break;
      const double part = lane + kWave * j < E ? exp(val[j] - mx) : 0.0;
      total += wave_sum(part);
    }
  }
  if (lane < K) {
    idx[(size_t)t * K + lane] = my_e;
    wout[(size_t)t * K + lane] = (float)(exp(v - mx) / total);
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

// bf16 -> fp32 (exact: the bf16 bits are the fp32 value's high half), eight
// values per thread; n is a multiple of 8 and both pointers 16-byte aligned
__global__ void __launch_bounds__(256) k_bf16_widen(const uint16_t* __restrict__ x, float* __restrict__ y,
                                                    int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const uint4 v = reinterpret_cast<const uint4*>(x)[i];
  float4* o = reinterpret_cast<float4*>(y) + 2 * i;
  o[0] = make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                     __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
  o[1] = make_float4(__uint_as_float(v.z << 16), __uint_as_float(v.z & 0xFFFF0000u),
                     __uint_as_float(v.w << 16), __uint_as_float(v.w & 0xFFFF0000u));
}

int launch_bf16_widen(const uint16_t* x, float* y, int64_t n, hipStream_t s) {
  const int64_t n8 = n / 8;
  if (n8 == 0) return 0;
  hipLaunchKernelGGL(k_bf16_widen, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, x, y, n8);
  return 0;
}

int launch_qdequant(const QT& W, uint8_t* codes, float* deq, hipStream_t s) {
  const int wpr = W.cols * W.bits / 32;
  const int64_t words = (int64_t)W.batch * W.rows * wpr;
  if (words == 0) return 0;
  const int64_t want = (words + 255) / 256;
  const int blocks = (int)(want < 65536 ? want : 65536);
  if (W.mode == 1) {
    hipLaunchKernelGGL(k_qdequant_mx, dim3(blocks), dim3(256), 0, s, W.q,
                       reinterpret_cast<const uint8_t*>(W.scales), words, wpr, W.cols, codes, deq);
    return 0;
  }
  MOEQ_BITS_LAUNCH(W.bits, k_qdequant, dim3(blocks), s, W.q, W.scales, W.biases, words, wpr,
                   W.cols, W.group_size, codes, deq);
  return 0;
}

// RMSNorm of one row per block (flash-moe-inference skill page, the two-pass
// rms_norm_pass1/2: the row's sum of squares, then every element scaled):
// h = x * r * g with r = 1/sqrt(mean(x^2) + eps), the mean square reduced in
// fp32 over the block and r taken in fp64.  H % 4 == 0.
__global__ __launch_bounds__(256) void k_rmsnorm(const float* __restrict__ x, int H,
                                                  const float* __restrict__ g, float eps,
                                                  float* __restrict__ h) {
  __shared__ float part[256 / kWave];
  __shared__ float s_r;
  const int t = blockIdx.x, tid = threadIdx.x;
  const float4* xr = reinterpret_cast<const float4*>(x + (size_t)t * H);
  float ss = 0.f;
  for (int i = tid; i < H / 4; i += 256) {
    const float4 v = xr[i];
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  if ((tid & (kWave - 1)) == 0) part[tid / kWave] = ss;
  __syncthreads();
  if (tid == 0) {
    float tot = 0.f;
    for (int w = 0; w < 256 / kWave; ++w) tot += part[w];
    s_r = (float)(1.0 / sqrt((double)tot / H + (double)eps));
  }
  __syncthreads();
  const float r = s_r;
  const float4* g4 = reinterpret_cast<const float4*>(g);
  float4* hr = reinterpret_cast<float4*>(h + (size_t)t * H);
  for (int i = tid; i < H / 4; i += 256) {
    const float4 v = xr[i], w = g4[i];
    hr[i] = make_float4(v.x * r * w.x, v.y * r * w.y, v.z * r * w.z, v.w * r * w.w);
  }
}

int launch_rmsnorm(const float* x, int M, int H, const float* g, float eps, float* h, hipStream_t s) {
  hipLaunchKernelGGL(k_rmsnorm, dim3(M), dim3(256), 0, s, x, H, g, eps, h);
  return 0;
}

int launch_qmatvec(const QT& W, const float* x, int M, float* y, hipStream_t s) {
  const int blocks = (W.rows + 3) / 4;
  if (W.mode == 1) {
    hipLaunchKernelGGL(k_qmatvec_mx, dim3(blocks), dim3(256), 0, s, W.q,
                       reinterpret_cast<const uint8_t*>(W.scales), W.rows, W.cols, x, M, y);
    return 0;
  }
  MOEQ_BITS_LAUNCH(W.bits, k_qmatvec, dim3(blocks), s, W.q, W.scales, W.biases, W.rows, W.cols,
                   W.group_size, x, M, y);
  return 0;
}

constexpr size_t kRouteCtrBytes = sizeof(int) * kLineInts * (1 + kFan);

size_t route_ctr_bytes() { return (kRouteCtrBytes + 255) / 256 * 256; }

// [counters][fp64 logits]: the counters sit at the same place for every M
size_t route_ws_bytes(int M, int E) {
  const size_t parts = M >= kMmaMinM ? (size_t)router_splits(M, E) : 1;
  return route_ctr_bytes() + ((sizeof(double) * parts * (size_t)M * E + 255) / 256) * 256;
}

int launch_route(const QT* router, const float* x_or_logits, int M, int E, int K, int renorm,
                 int32_t* idx, float* w, float* logits32, void* ws, hipStream_t s) {
  char* b = reinterpret_cast<char*>(ws);
  return launch_route_parts(router, x_or_logits, M, E, K, renorm, idx, w, logits32,
                            b ? reinterpret_cast<double*>(b + route_ctr_bytes()) : nullptr,
                            reinterpret_cast<int*>(b), s);
}

// Router projection for many tokens with the tokens' x staged in LDS: a block
// takes kRtTok tokens and kRtRows router rows (kRtRows / 4 per wave), so one
// LDS read of x feeds every row of the wave and a block reads its tokens' x
// from memory once (one wave per row re-reads x from L2 for every row).  The
// arithmetic is k_router's: each fp32 dequantized weight widened exactly,
// fp64 products and sums (per lane over its chunks in order, then the wave).
// H <= 4096 (x of kRtTok tokens within 64 KB).
// Router projection for many tokens on the fp64 matrix cores
// (v_mfma_f64_16x16x4f64): a wave takes 16 tokens x 16 router rows over one
// split of the hidden dimension, in 64-column chunks.  Lane (i, q), i = lane
// % 16, q = lane / 16, feeds token i's x and row i's weights for columns
// 64c + 16q + s, s = 0..15, one column per instruction, the weight the fp32
// scale * code + bias widened exactly (as in the other router kernels); the
// products are exact in fp64 and summed in fp64.  Each split's sums go to
// part[split][token][row]; the top-K kernel adds the splits in order.
// H % 64 == 0.
template <int BITS>
__global__ void __launch_bounds__(kRouteThreads) k_router_mma(QT W, const float* __restrict__ x,
                                                              int M, int nsplit,
                                                              double* __restrict__ part) {
  typedef double f64x4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int rows = W.rows, H = W.cols;
  const int n0 = (blockIdx.x * (kRouteThreads / kWave) + wid) * 16;   // the wave's router rows
  const int m0 = blockIdx.y * 16;                                     // its tokens
  const int sp = blockIdx.z;
  const int nchunk = H / 64;
  const int c0 = sp * nchunk / nsplit, c1 = (sp + 1) * nchunk / nsplit;
  const int i = lane & 15, q = lane >> 4;
  // rows and tokens past the ends re-read the last valid one (never stored)
  const int r = min(n0 + i, rows - 1);
  const int t = min(m0 + i, M - 1);
  const float* xt = x + (size_t)t * H;
  const uint32_t* wq = W.q + (size_t)r * (H / (32 / BITS));
  const uint16_t* ws = W.scales + (size_t)r * (H / W.group_size);
  const uint16_t* wb = W.biases + (size_t)r * (H / W.group_size);
  const int gsh = __builtin_ctz((unsigned)W.group_size);
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
  // a chunk's operands: the lane's 16 columns (one group) of codes, its
  // scale and bias, and the token's 16 x values; the next chunk's are loaded
  // while this one's products run
  struct Chunk {
    uint32_t cw[BITS / 2];
    uint32_t sb;
    float4 xv[4];
  };
  auto load = [&](int c, Chunk& C) {
    const int k0 = min(c, c1 - 1) * 64 + 16 * q;   // clamped: always a valid address
#pragma unroll
    for (int u = 0; u < BITS / 2; ++u) C.cw[u] = wq[k0 / (32 / BITS) + u];
    C.sb = (uint32_t)ws[k0 >> gsh] | ((uint32_t)wb[k0 >> gsh] << 16);
#pragma unroll
    for (int u = 0; u < 4; ++u) C.xv[u] = reinterpret_cast<const float4*>(xt + k0)[u];
  };
  Chunk cur, nxt;
  if (c0 < c1) load(c0, cur);
  for (int c = c0; c < c1; ++c) {
    load(c + 1, nxt);
    const float sc = bf16_to_f32(cur.sb & 0xFFFFu), bi = bf16_to_f32(cur.sb >> 16);
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) {
      constexpr int kPer = 32 / BITS;
      const uint32_t code = (cur.cw[s2 / kPer] >> (BITS * (s2 % kPer))) & ((1u << BITS) - 1u);
      const double w = (double)fmaf(sc, (float)code, bi);
      const float4 x4v = cur.xv[s2 / 4];
      const float xs = (s2 & 3) == 0 ? x4v.x : (s2 & 3) == 1 ? x4v.y : (s2 & 3) == 2 ? x4v.z : x4v.w;
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xs, w, acc, 0, 0, 0);
    }
    cur = nxt;
  }
  // accumulator: register v of lane (i, q) holds token 4v + q of row i (the
  // instruction's output rows interleave over the four lane groups)
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int tok = m0 + 4 * v + q, row = n0 + i;
    if (tok < M && row < rows) part[((size_t)sp * M + tok) * rows + row] = acc[v];
  }
}

constexpr int kRtTok = 4;
constexpr int kRtRows = 16;
template <int BITS>
__global__ void __launch_bounds__(kRouteThreads) k_router_tile(QT W, const float* __restrict__ x,
                                                               int M, double* __restrict__ logits,
                                                               float* __restrict__ logits32) {
  extern __shared__ __attribute__((aligned(16))) float xs[];   // [kRtTok][H], chunk-interleaved
  constexpr int kCpc = 128 / BITS;
  constexpr int kRpw = kRtRows / (kRouteThreads / kWave);     // rows per wave
  constexpr int kCpl = 4096 / kCpc / kWave;                   // chunks per lane at most (H <= 4096)
  const int rows = W.rows, H = W.cols;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int r0 = blockIdx.x * kRtRows + wid * kRpw;
  const int m0 = blockIdx.y * kRtTok;
  const int nm = min(kRtTok, M - m0);
  const int nch = H / kCpc;
  const int groups = H / W.group_size;
  const int gsh = __builtin_ctz((unsigned)W.group_size);
  // every weight load of the lane first (clamped, always valid addresses;
  // rows past the last re-read row 0 and are never stored), so they are in
  // flight while x is staged
  uint4 wv[kCpl][kRpw];
  uint32_t wsb[kCpl][kRpw];                   // bf16 scale | bias << 16
#pragma unroll
  for (int j = 0; j < kCpl; ++j) {
    const int c = min(lane + kWave * j, nch - 1);
    const int g = (c * kCpc) >> gsh;
#pragma unroll
    for (int rr = 0; rr < kRpw; ++rr) {
      const int r = r0 + rr < rows ? r0 + rr : 0;
      wv[j][rr] = reinterpret_cast<const uint4*>(W.q + (size_t)r * (H / (32 / BITS)))[c];
      wsb[j][rr] = (uint32_t)W.scales[(size_t)r * groups + g] |
                   ((uint32_t)W.biases[(size_t)r * groups + g] << 16);
    }
  }
  // x of the block's tokens (tokens past the last re-read the first): float4
  // f of chunk c of token t at t * H / 4 + f * nch + c
  float4* x4 = reinterpret_cast<float4*>(xs);
  for (int i = tid; i < kRtTok * (H / 4); i += kRouteThreads) {
    const int t = i / (H / 4), ii = i - t * (H / 4);
    const int m = m0 + (t < nm ? t : 0);
    x4[t * (H / 4) + (ii % (kCpc / 4)) * nch + ii / (kCpc / 4)] =
        reinterpret_cast<const float4*>(x + (size_t)m * H)[ii];
  }
  __syncthreads();
  double acc[kRpw][kRtTok];
#pragma unroll
  for (int rr = 0; rr < kRpw; ++rr)
#pragma unroll
    for (int t = 0; t < kRtTok; ++t) acc[rr][t] = 0.0;
#pragma unroll
  for (int j = 0; j < kCpl; ++j) {
    const int c = lane + kWave * j;
    if (c < nch) {
#pragma unroll
      for (int f = 0; f < kCpc / 4; ++f) {
        double xd[kRtTok][4];                // widened once, used by every row of the wave
#pragma unroll
        for (int t = 0; t < kRtTok; ++t) {
          const float4 xv = x4[t * (H / 4) + f * nch + c];
          xd[t][0] = (double)xv.x;
          xd[t][1] = (double)xv.y;
          xd[t][2] = (double)xv.z;
          xd[t][3] = (double)xv.w;
        }
#pragma unroll
        for (int rr = 0; rr < kRpw; ++rr) {
          const float sc = bf16_to_f32(wsb[j][rr] & 0xFFFFu), bi = bf16_to_f32(wsb[j][rr] >> 16);
          double w[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            w[q] = (double)fmaf(sc, (float)chunk_code<BITS>(wv[j][rr], 4 * f + q), bi);
#pragma unroll
          for (int t = 0; t < kRtTok; ++t) {
            acc[rr][t] = fma(w[0], xd[t][0], acc[rr][t]);
            acc[rr][t] = fma(w[1], xd[t][1], acc[rr][t]);
            acc[rr][t] = fma(w[2], xd[t][2], acc[rr][t]);
            acc[rr][t] = fma(w[3], xd[t][3], acc[rr][t]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int rr = 0; rr < kRpw; ++rr) {
#pragma unroll
    for (int t = 0; t < kRtTok; ++t) {
      const double a = wave_sum(acc[rr][t]);
      const int r = r0 + rr;
      if (lane == 0 && t < nm && r < rows) {
        logits[(size_t)(m0 + t) * rows + r] = a;
        if (logits32) logits32[(size_t)(m0 + t) * rows + r] = (float)a;
      }
    }
  }
}

int launch_route_parts(const QT* router, const float* x_or_logits, int M, int E, int K, int renorm,
                       int32_t* idx, float* w, float* logits32, double* l64, int* ctr,
                       hipStream_t s) {
  const dim3 grid_topk((M + kRouteThreads / kWave - 1) / (kRouteThreads / kWave));
  // the many-token top-K with the fewest key slots per lane that hold E
  auto topk = [&](const double* l64_, const float* l32_, int nparts, float* l32_out) {
#define MOEQ_TOPK(P_)                                                                             \
  hipLaunchKernelGGL(k_topk_wave<P_>, grid_topk, dim3(kRouteThreads), 0, s, l64_, l32_, M, E, K,  \
                     renorm, idx, w, nparts, l32_out)
    if (E <= 64) MOEQ_TOPK(1);
    else if (E <= 128) MOEQ_TOPK(2);
    else if (E <= 256) MOEQ_TOPK(4);
    else if (E <= 512) MOEQ_TOPK(8);
    else MOEQ_TOPK(16);
#undef MOEQ_TOPK
  };
  static_assert(kMaxE <= 16 * kWave, "k_topk_wave holds at most 16 keys per lane");
  if (!router) {
    topk(nullptr, x_or_logits, 1, nullptr);
    return 0;
  }
  const dim3 grid((E + 3) / 4);
  const QT& W = *router;
  const bool last = M <= kLastTopkMaxM;
  const dim3 grid_many((E + 3) / 4, (M + kRouteTM - 1) / kRouteTM);
  // many tokens: the LDS-staged tile kernel when the tokens' x fits (64 KB)
  const bool tile = W.cols <= 4096;
  const size_t tile_lds = sizeof(float) * kRtTok * (size_t)W.cols;
  const dim3 grid_tile((E + kRtRows - 1) / kRtRows, (M + kRtTok - 1) / kRtTok);
  // the fp64 matrix cores from 16 tokens (hidden a multiple of 64)
  const bool mma = !last && M >= kMmaMinM && W.cols % 64 == 0;
  const int nsplit = mma ? min(router_splits(M, E), W.cols / 64) : 1;
  const dim3 grid_mma((E + 63) / 64, (M + 15) / 16, nsplit);
#define MOEQ_ROUTER(B_)                                                                           \
  if (W.bits == B_) {                                                                             \
    if (last)                                                                                     \
      hipLaunchKernelGGL((k_router<B_, true>), grid, dim3(kRouteThreads), 0, s, W, x_or_logits, M, \
                         K, renorm, l64, ctr, logits32, idx, w);                                   \
    else if (mma)                                                                                 \
      hipLaunchKernelGGL((k_router_mma<B_>), grid_mma, dim3(kRouteThreads), 0, s, W, x_or_logits, \
                         M, nsplit, l64);                                                          \
    else if (tile)                                                                                \
      hipLaunchKernelGGL((k_router_tile<B_>), grid_tile, dim3(kRouteThreads), tile_lds, s, W,     \
                         x_or_logits, M, l64, logits32);                                          \
    else                                                                                          \
      hipLaunchKernelGGL((k_router_many<B_>), grid_many, dim3(kRouteThreads), 0, s, W,            \
                         x_or_logits, M, l64, logits32);                                          \
  }
  MOEQ_ROUTER(8)
  MOEQ_ROUTER(4)
  MOEQ_ROUTER(2)
#undef MOEQ_ROUTER
  if (!last) topk(l64, nullptr, mma ? nsplit : 1, mma ? logits32 : nullptr);
  return 0;
}

}  // namespace moeq
