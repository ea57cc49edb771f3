// Gather GEMMs of the prefill path on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16).
//
// ml-explore/mlx issue #3856 (minimal repro: gather_qmm with rhs_indices,
// transpose=True) defines the product; its row-count defect is why every tile
// here carries its exact row count in int32, rows past it are zero-filled on
// load and never stored.
//
// A block computes a 256-row x 128-column tile of one expert: 256 rows
// gathered through the sorted pair list, 128 weight rows ("B columns").  Per
// 64-wide reduction step (one quantization group) it stages the A rows as bf16
// in LDS and dequantizes the B codes to bf16 in LDS (w = scale*code + bias,
// rounded to nearest even), while the next step's global loads are in flight;
// four waves each own a 128x64 sub-tile (4x2 MFMA 32x32 tiles).  Dequantizing
// once per 256 rows keeps the VALU work well under the MFMA time.
//
// Tile order is XCD-aware: workgroups are dealt round-robin to the 8 XCDs, so
// block b works on item (b % 8) * ceil(T/8) + b / 8 of the T (m-tile, n-tile)
// items in m-major order: all n-tiles of an m-tile run on one XCD back to back
// and the gathered A rows are re-read from that XCD's L2, not from HBM.
//
// Modes: 0 plain   out[pair][n] = x[pair] . W_e[n]                 (fp32)
//        1 gate/up h[sorted row][i] = silu(x.G_e[i]) * (x.U_e[i])  (bf16)
//        2 down    ypair[pair][n] = w_pair * (h[sorted row] . D_e[n]) (bf16)
#include "common.h"
#include "launch.h"

namespace moeq {

typedef short bf16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kBM = kGemmBM;  // 256 rows
constexpr int kBN = 128;      // B columns per block
constexpr int kBK = 64;       // one group per k-step
constexpr int kLds = kBK + 8; // padded row stride (bf16 elements): 144 B, conflict-free b128 reads
constexpr int kThreads = 256;
constexpr int kXcd = 8;

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};   // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// dequantize 32 codes (this thread's half of a 64-code group) to 16 packed bf16 pairs
template <int BITS>
__device__ __forceinline__ void dequant32(const uint4* v, float s, float b, uint32_t* out) {
  if constexpr (BITS == 8) {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t x = w < 4 ? (&v[0].x)[w] : (&v[1].x)[w - 4];
      out[2 * w] = pack_bf16(fmaf(s, (float)(x & 0xFFu), b), fmaf(s, (float)((x >> 8) & 0xFFu), b));
      out[2 * w + 1] = pack_bf16(fmaf(s, (float)((x >> 16) & 0xFFu), b), fmaf(s, (float)(x >> 24), b));
    }
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x = (&v[0].x)[w];
#pragma unroll
      for (int j = 0; j < 8; j += 2)
        out[4 * w + j / 2] = pack_bf16(fmaf(s, (float)((x >> (4 * j)) & 0xFu), b),
                                       fmaf(s, (float)((x >> (4 * j + 4)) & 0xFu), b));
    }
  } else {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const uint32_t x = (&v[0].x)[w];
#pragma unroll
      for (int j = 0; j < 16; j += 2)
        out[8 * w + j / 2] = pack_bf16(fmaf(s, (float)((x >> (2 * j)) & 0x3u), b),
                                       fmaf(s, (float)((x >> (2 * j + 2)) & 0x3u), b));
    }
  }
}

template <int BITS>
__device__ __forceinline__ void load_codes(uint4* v, const uint32_t* p) {
  if constexpr (BITS == 8) {
    v[0] = reinterpret_cast<const uint4*>(p)[0];
    v[1] = reinterpret_cast<const uint4*>(p)[1];
  } else if constexpr (BITS == 4) {
    v[0] = reinterpret_cast<const uint4*>(p)[0];
  } else {
    const uint2 t = reinterpret_cast<const uint2*>(p)[0];
    v[0] = make_uint4(t.x, t.y, 0u, 0u);
  }
}

template <int BITS, int MODE>
__global__ void __launch_bounds__(kThreads, 2) k_gqmm(QT W, QT W2, int N, int Kd,
                                                      const uint16_t* __restrict__ A, int a_div,
                                                      GatherWs ws, const float* __restrict__ wts,
                                                      void* __restrict__ out, int ntn) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kBN * kLds];
  __shared__ int s_pair[kBM];
  __shared__ float s_w[kBM];

  // ---- XCD-aware item: block b -> item (b % 8) * ceil(T/8) + b / 8
  const int T = ws.n_tiles[0] * ntn;
  const int per = (T + kXcd - 1) / kXcd;
  const int item = (blockIdx.x % kXcd) * per + blockIdx.x / kXcd;
  if (blockIdx.x / kXcd >= per || item >= T) return;
  const int tile = item / ntn;
  const int nt = item - tile * ntn;
  const int4 Tl = ws.tiles[tile];
  const int e = Tl.x, row0 = Tl.y, rows = Tl.z;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int wm = wid & 1, wn = wid >> 1;

  for (int r = tid; r < kBM; r += kThreads) {
    const int pair = r < rows ? ws.sorted[row0 + r] : 0;
    s_pair[r] = pair;
    if (MODE == 2) s_w[r] = r < rows ? wts[pair] : 0.f;
  }
  __syncthreads();

  // ---- A source rows: rows (tid>>3) + 32u (u < 8), 16-byte segment tid&7
  const int aseg = tid & 7;
  const uint16_t* asrc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int r = (tid >> 3) + 32 * u;
    asrc[u] = nullptr;
    if (r < rows) asrc[u] = MODE == 2 ? A + (size_t)(row0 + r) * Kd : A + (size_t)(s_pair[r] / a_div) * Kd;
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
      n = nt * 64 + cw * 32 + j;
      if (hf) M = &W2;
    } else {
      n = nt * kBN + bc;
    }
    if (n < N) {
      const size_t row = (size_t)e * N + n;
      bq = M->q + row * (Kd / (32 / BITS)) + bh * BITS;  // 32 codes = BITS words
      bs = M->scales + row * (Kd / kGroup);
      bb = M->biases + row * (Kd / kGroup);
    }
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 areg[8];
  uint4 breg[2];
  float bsv = 0.f, bbv = 0.f;
  const int ksteps = Kd / kBK;

  auto gload = [&](int kt) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      areg[u] = asrc[u] ? *reinterpret_cast<const uint4*>(asrc[u] + kt * kBK + aseg * 8)
                        : make_uint4(0, 0, 0, 0);
    if (bq) {
      load_codes<BITS>(breg, bq + (size_t)kt * (kBK / (32 / BITS)));
      bsv = bf16_to_f32(bs[kt]);
      bbv = bf16_to_f32(bb[kt]);
    }
  };

  gload(0);
  for (int kt = 0; kt < ksteps; ++kt) {
    // ---- registers -> LDS (B dequantized to bf16)
#pragma unroll
    for (int u = 0; u < 8; ++u)
      *reinterpret_cast<uint4*>(&As[((tid >> 3) + 32 * u) * kLds + aseg * 8]) = areg[u];
    {
      uint32_t packed[16];
      if (bq) {
        dequant32<BITS>(breg, bsv, bbv, packed);
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
    // ---- MFMA on the staged tile: 4 k16 steps x (4 x 2) tiles
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int kof = kk * 16 + 8 * (lane >> 5);
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        af[mi] = *reinterpret_cast<const bf16x8*>(&As[(wm * 128 + mi * 32 + (lane & 31)) * kLds + kof]);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bfr[ni] = *reinterpret_cast<const bf16x8*>(&Bs[(wn * 64 + ni * 32 + (lane & 31)) * kLds + kof]);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- epilogue.  32x32 accumulator layout: register r of lane l holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = wm * 128 + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (rl >= rows) continue;
      if (MODE == 1) {
        const int i = nt * 64 + wn * 32 + (lane & 31);
        const float h = silu(acc[mi][0][r]) * acc[mi][1][r];
        const bf16x2_t hv = {(__bf16)h, (__bf16)0.f};
        reinterpret_cast<uint16_t*>(out)[(size_t)(row0 + rl) * N + i] =
            (uint16_t)(__builtin_bit_cast(uint32_t, hv) & 0xFFFFu);
      } else {
        const int pair = s_pair[rl];
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int n = nt * kBN + wn * 64 + ni * 32 + (lane & 31);
          if (n < N) {
            if (MODE == 2) {
              const bf16x2_t v = {(__bf16)(acc[mi][ni][r] * s_w[rl]), (__bf16)0.f};
              reinterpret_cast<uint16_t*>(out)[(size_t)pair * N + n] =
                  (uint16_t)(__builtin_bit_cast(uint32_t, v) & 0xFFFFu);
            } else {
              reinterpret_cast<float*>(out)[(size_t)pair * N + n] = acc[mi][ni][r];
            }
          }
        }
      }
    }
  }
}

// y[t][c] = sum over slots k (in order) of ypair[t*K+k][c] (bf16 -> fp32); NaN
// for a pair whose expert index is out of range (its row was never computed).
__global__ void __launch_bounds__(256) k_combine(const uint16_t* __restrict__ ypair,
                                                 const int32_t* __restrict__ idx, int M, int K,
                                                 int H, int E, float* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // 8-column group
  const int64_t total = (int64_t)M * H / 8;
  if (i >= total) return;
  const int64_t t = (i * 8) / H;
  const int64_t c = i * 8 - t * H;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < K; ++k) {
    const int64_t p = t * K + k;
    const int e = idx[p];
    if (e >= 0 && e < E) {
      const uint4 v = *reinterpret_cast<const uint4*>(ypair + p * H + c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[2 * j] += bf16_to_f32(w[j] & 0xFFFFu);
        s[2 * j + 1] += bf16_to_f32(w[j] >> 16);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) s[j] = __builtin_nanf("");
    }
  }
  float4* yo = reinterpret_cast<float4*>(y + t * H + c);
  yo[0] = make_float4(s[0], s[1], s[2], s[3]);
  yo[1] = make_float4(s[4], s[5], s[6], s[7]);
}

__global__ void __launch_bounds__(256) k_mark_invalid(const int32_t* __restrict__ idx, int n, int E,
                                                      int N, float* __restrict__ out) {
  const int row = blockIdx.x;
  const int e = idx[row];
  if (e >= 0 && e < E) return;
  for (int c = threadIdx.x; c < N; c += blockDim.x) out[(size_t)row * N + c] = __builtin_nanf("");
}

#define MOEQ_GEMM_BITS(bits, MODE_, ...)                                                        \
  do {                                                                                         \
    if ((bits) == 8) hipLaunchKernelGGL((k_gqmm<8, MODE_>), __VA_ARGS__);                      \
    else if ((bits) == 4) hipLaunchKernelGGL((k_gqmm<4, MODE_>), __VA_ARGS__);                 \
    else hipLaunchKernelGGL((k_gqmm<2, MODE_>), __VA_ARGS__);                                  \
  } while (0)

static dim3 gemm_grid(const GatherWs& ws, int ntn) {
  const int items = ws.max_tiles * ntn;
  return dim3((unsigned)(((items + kXcd - 1) / kXcd) * kXcd));
}

int launch_gemm_gate_up(const QT& gate, const QT& up, const uint16_t* x, int K, const GatherWs& ws,
                        int n, hipStream_t s) {
  (void)n;
  const int I = gate.rows, H = gate.cols;
  const int ntn = I / 64;
  MOEQ_GEMM_BITS(gate.bits, 1, gemm_grid(ws, ntn), dim3(kThreads), 0, s, gate, up, I, H, x, K, ws,
                 (const float*)nullptr, (void*)ws.h, ntn);
  return 0;
}

int launch_gemm_down(const QT& down, const float* w, const GatherWs& ws, int n, hipStream_t s) {
  (void)n;
  const int H = down.rows, I = down.cols;
  const int ntn = (H + kBN - 1) / kBN;
  MOEQ_GEMM_BITS(down.bits, 2, gemm_grid(ws, ntn), dim3(kThreads), 0, s, down, down, H, I,
                 (const uint16_t*)ws.h, 1, ws, w, (void*)ws.ypair, ntn);
  return 0;
}

int launch_gemm_plain(const QT& W, const uint16_t* x, float* out, const GatherWs& ws, int n,
                      hipStream_t s) {
  (void)n;
  const int ntn = (W.rows + kBN - 1) / kBN;
  MOEQ_GEMM_BITS(W.bits, 0, gemm_grid(ws, ntn), dim3(kThreads), 0, s, W, W, W.rows, W.cols, x, 1, ws,
                 (const float*)nullptr, (void*)out, ntn);
  return 0;
}

int launch_mark_invalid_rows(const int32_t* idx, int n, int E, int N, float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_mark_invalid, dim3(n), dim3(256), 0, s, idx, n, E, N, out);
  return 0;
}

int launch_combine(const uint16_t* ypair, const int32_t* idx, int M, int K, int H, int E, float* y,
                   hipStream_t s) {
  const int64_t total = (int64_t)M * H / 8;
  if (total == 0) return 0;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)blocks), dim3(256), 0, s, ypair, idx, M, K, H, E, y);
  return 0;
}

}  // namespace moeq
