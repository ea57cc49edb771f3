// Gather GEMMs of the prefill path on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16).
//
// A tile covers 128 rows of one expert (rows gathered through the sorted pair
// list) and 128 weight rows ("B columns").  Per 64-wide reduction step (one
// quantization group) the block stages the A rows as bf16 in LDS and
// dequantizes the B codes to bf16 in LDS (w = scale*code + bias, then
// round-to-nearest-even), and four waves each run a 64x64 sub-tile as 2x2
// MFMA 32x32x16 tiles over four k-steps.  ml-explore/mlx issue #3856
// (minimal repro: gather_qmm with rhs_indices, transpose=True) defines the
// product; its row-count defect is why every tile carries its exact row count
// in int32 and rows past it are zero-filled on load and never stored.
//
// Modes: 0 plain   out[pair][n] = x[pair] . W_e[n]                 (fp32)
//        1 gate/up h[sorted row][i] = silu(x.G_e[i]) * (x.U_e[i])  (bf16)
//        2 down    ypair[pair][n] = w_pair * (h[sorted row] . D_e[n]) (fp32)
#include "common.h"
#include "launch.h"

namespace moeq {

typedef short bf16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

constexpr int kBM = kGemmBM;  // 128 rows
constexpr int kBN = 128;      // B columns per block
constexpr int kBK = 64;       // one group per k-step
constexpr int kLds = kBK + 8; // padded row stride (bf16 elements): 144 B

template <int BITS>
struct BLoad;  // per-thread share of one (column, half-group): 32 codes
template <>
struct BLoad<8> { uint4 v[2]; };
template <>
struct BLoad<4> { uint4 v[1]; };
template <>
struct BLoad<2> { uint2 v[1]; };

template <int BITS>
__device__ __forceinline__ void load_b(BLoad<BITS>& d, const uint32_t* p) {
  if constexpr (BITS == 8) {
    d.v[0] = reinterpret_cast<const uint4*>(p)[0];
    d.v[1] = reinterpret_cast<const uint4*>(p)[1];
  } else if constexpr (BITS == 4) {
    d.v[0] = reinterpret_cast<const uint4*>(p)[0];
  } else {
    d.v[0] = reinterpret_cast<const uint2*>(p)[0];
  }
}

template <int BITS>
__device__ __forceinline__ uint32_t b_word(const BLoad<BITS>& d, int w) {
  if constexpr (BITS == 8) {
    const uint4& v = d.v[w >> 2];
    const int k = w & 3;
    return k == 0 ? v.x : (k == 1 ? v.y : (k == 2 ? v.z : v.w));
  } else if constexpr (BITS == 4) {
    return w == 0 ? d.v[0].x : (w == 1 ? d.v[0].y : (w == 2 ? d.v[0].z : d.v[0].w));
  } else {
    return w == 0 ? d.v[0].x : d.v[0].y;
  }
}

template <int BITS, int MODE>
__global__ void __launch_bounds__(256) k_gqmm(QT W, QT W2, int N, int Kd,
                                              const uint16_t* __restrict__ A, int a_div,
                                              GatherWs ws, const float* __restrict__ wts,
                                              void* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kBN * kLds];

  const int tile = blockIdx.x;
  if (tile >= ws.n_tiles[0]) return;
  const int4 T = ws.tiles[tile];
  const int e = T.x, row0 = T.y, rows = T.z;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int wm = wid & 1, wn = wid >> 1;

  // ---- A source rows of this thread: rows (tid>>3) + 32u, 16-byte segment tid&7
  const int aseg = tid & 7;
  const uint16_t* asrc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = (tid >> 3) + 32 * u;
    asrc[u] = nullptr;
    if (r < rows) {
      if (MODE == 2) {
        asrc[u] = A + (size_t)(row0 + r) * Kd;
      } else {
        const int pair = ws.sorted[row0 + r];
        asrc[u] = A + (size_t)(pair / a_div) * Kd;
      }
    }
  }

  // ---- B column of this thread: column bc = tid>>1, codes [32*bh, 32*bh+32) of each group
  const int bc = tid >> 1, bh = tid & 1;
  const uint32_t* bq = nullptr;
  const uint16_t *bs = nullptr, *bb = nullptr;
  {
    int n;
    const QT* M = &W;
    if (MODE == 1) {
      const int cw = bc >> 6, hf = (bc >> 5) & 1, j = bc & 31;
      n = blockIdx.y * 64 + cw * 32 + j;
      if (hf) M = &W2;
    } else {
      n = blockIdx.y * kBN + bc;
    }
    if (n < N) {
      const size_t row = (size_t)e * N + n;
      bq = M->q + row * (Kd / (32 / BITS)) + bh * (BITS);  // 32 codes = BITS words
      bs = M->scales + row * (Kd / kGroup);
      bb = M->biases + row * (Kd / kGroup);
    }
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 areg[4];
  BLoad<BITS> breg;
  float bsv = 0.f, bbv = 0.f;
  const int ksteps = Kd / kBK;

  auto gload = [&](int kt) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      areg[u] = asrc[u] ? *reinterpret_cast<const uint4*>(asrc[u] + kt * kBK + aseg * 8)
                        : make_uint4(0, 0, 0, 0);
    if (bq) {
      load_b<BITS>(breg, bq + (size_t)kt * (kBK / (32 / BITS)));
      bsv = bf16_to_f32(bs[kt]);
      bbv = bf16_to_f32(bb[kt]);
    }
  };

  gload(0);
  for (int kt = 0; kt < ksteps; ++kt) {
    // ---- registers -> LDS (B dequantized to bf16)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      *reinterpret_cast<uint4*>(&As[((tid >> 3) + 32 * u) * kLds + aseg * 8]) = areg[u];
    {
      uint32_t packed[16];
      if (bq) {
        constexpr int kPer = 32 / BITS;
        constexpr uint32_t kMask = (1u << BITS) - 1u;
#pragma unroll
        for (int j = 0; j < 32; j += 2) {
          const uint32_t w0 = b_word<BITS>(breg, j / kPer);
          const uint32_t c0 = (w0 >> (BITS * (j % kPer))) & kMask;
          const uint32_t c1 = (w0 >> (BITS * ((j + 1) % kPer))) & kMask;
          const uint32_t lo = f32_to_bf16_rne(fmaf(bsv, (float)c0, bbv));
          const uint32_t hi = f32_to_bf16_rne(fmaf(bsv, (float)c1, bbv));
          packed[j / 2] = lo | (hi << 16);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) packed[j] = 0u;
      }
      uint4* dst = reinterpret_cast<uint4*>(&Bs[bc * kLds + bh * 32]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        dst[q] = make_uint4(packed[4 * q], packed[4 * q + 1], packed[4 * q + 2], packed[4 * q + 3]);
    }
    __syncthreads();
    if (kt + 1 < ksteps) gload(kt + 1);
    // ---- MFMA on the staged tile
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int kof = kk * 16 + 8 * (lane >> 5);
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        af[mi] = *reinterpret_cast<const bf16x8*>(&As[(wm * 64 + mi * 32 + (lane & 31)) * kLds + kof]);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bfr[ni] = *reinterpret_cast<const bf16x8*>(&Bs[(wn * 64 + ni * 32 + (lane & 31)) * kLds + kof]);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- epilogue.  32x32 accumulator layout: register r of lane l holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (rl >= rows) continue;
      if (MODE == 1) {
        const int i = blockIdx.y * 64 + wn * 32 + (lane & 31);
        const float h = silu(acc[mi][0][r]) * acc[mi][1][r];
        reinterpret_cast<uint16_t*>(out)[(size_t)(row0 + rl) * N + i] = (uint16_t)f32_to_bf16_rne(h);
      } else {
        const int pair = ws.sorted[row0 + rl];
        const float scale = MODE == 2 ? wts[pair] : 1.0f;
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int n = blockIdx.y * kBN + wn * 64 + ni * 32 + (lane & 31);
          if (n < N) reinterpret_cast<float*>(out)[(size_t)pair * N + n] = acc[mi][ni][r] * scale;
        }
      }
    }
  }
}

// y[t][c] = sum over slots k (in order) of ypair[t*K+k][c]; NaN for a pair
// whose expert index is out of range (its row was never computed).
__global__ void __launch_bounds__(256) k_combine(const float* __restrict__ ypair,
                                                 const int32_t* __restrict__ idx, int M, int K,
                                                 int H, int E, float* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // float4 index
  const int64_t total = (int64_t)M * H / 4;
  if (i >= total) return;
  const int64_t t = (i * 4) / H;
  const int64_t c = i * 4 - t * H;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = 0; k < K; ++k) {
    const int64_t p = t * K + k;
    const int e = idx[p];
    float4 v;
    if (e >= 0 && e < E) v = *reinterpret_cast<const float4*>(ypair + p * H + c);
    else v = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""));
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  *reinterpret_cast<float4*>(y + t * H + c) = s;
}

__global__ void __launch_bounds__(256) k_mark_invalid(const int32_t* __restrict__ idx, int n, int E,
                                                      int N, float* __restrict__ out) {
  const int row = blockIdx.x;
  const int e = idx[row];
  if (e >= 0 && e < E) return;
  for (int c = threadIdx.x; c < N; c += blockDim.x) out[(size_t)row * N + c] = __builtin_nanf("");
}

#define MOEQ_GEMM_BITS(bits, MODE_, ...)                                                         \
  do {                                                                                          \
    if ((bits) == 8) hipLaunchKernelGGL((k_gqmm<8, MODE_>), __VA_ARGS__);                       \
    else if ((bits) == 4) hipLaunchKernelGGL((k_gqmm<4, MODE_>), __VA_ARGS__);                  \
    else hipLaunchKernelGGL((k_gqmm<2, MODE_>), __VA_ARGS__);                                   \
  } while (0)

int launch_gemm_gate_up(const QT& gate, const QT& up, const uint16_t* x, int K, const GatherWs& ws,
                        int n, hipStream_t s) {
  (void)n;
  const int I = gate.rows, H = gate.cols;
  dim3 grid(ws.max_tiles, I / 64);
  MOEQ_GEMM_BITS(gate.bits, 1, grid, dim3(256), 0, s, gate, up, I, H, x, K, ws,
                 (const float*)nullptr, (void*)ws.h);
  return 0;
}

int launch_gemm_down(const QT& down, const float* w, const GatherWs& ws, int n, hipStream_t s) {
  (void)n;
  const int H = down.rows, I = down.cols;
  dim3 grid(ws.max_tiles, (H + kBN - 1) / kBN);
  MOEQ_GEMM_BITS(down.bits, 2, grid, dim3(256), 0, s, down, down, H, I, (const uint16_t*)ws.h, 1, ws,
                 w, (void*)ws.ypair);
  return 0;
}

int launch_gemm_plain(const QT& W, const uint16_t* x, float* out, const GatherWs& ws, int n,
                      hipStream_t s) {
  (void)n;
  dim3 grid(ws.max_tiles, (W.rows + kBN - 1) / kBN);
  MOEQ_GEMM_BITS(W.bits, 0, grid, dim3(256), 0, s, W, W, W.rows, W.cols, x, 1, ws,
                 (const float*)nullptr, (void*)out);
  return 0;
}

int launch_mark_invalid_rows(const int32_t* idx, int n, int E, int N, float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_mark_invalid, dim3(n), dim3(256), 0, s, idx, n, E, N, out);
  return 0;
}

int launch_combine(const float* ypair, const int32_t* idx, int M, int K, int H, int E, float* y,
                   hipStream_t s) {
  const int64_t total = (int64_t)M * H / 4;
  if (total == 0) return 0;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)blocks), dim3(256), 0, s, ypair, idx, M, K, H, E, y);
  return 0;
}

}  // namespace moeq
