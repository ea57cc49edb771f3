// Batched decode (fp32 activations, many tokens per call): the expert part of
// the step with every touched expert's weights streamed once for all the
// tokens routed to it.
//
// The step per selected expert is the one of the decode path (markbaseengine
// MOE_ROUTER_WORKS_BREAKTHROUGH, "Forward Pass Sequence"; flash-moe-inference
// kernels swiglu and moe_combine_residual).  With M tokens and top-K routing
// an expert serves r_e of the M*K (token, slot) pairs, so per token the
// decode launch would stream each expert r_e times (and the shared expert M
// times).  Here the pairs are grouped by expert first (the sort of the
// gather path, tiles of at most kBTile rows), then
//   k_bgate   one unit = (tile, 16 gate/up rows): the rows are loaded once,
//             kept in registers and applied to the tile's tokens kBTok at a
//             time (x staged in LDS), SwiGLU, h[pair]; the shared expert is one
//             tile holding all M tokens, and its first row block also computes
//             the shared_expert_gate logits;
//   k_bdown   one unit = (tile, 8*64/LPR output rows): down rows loaded once,
//             applied to the tile's h kBTok pairs at a time, scaled by the
//             routing weight (or the sigmoid of the shared gate) into a per-pair
//             output row;
//   k_bcombine y[t] = sum over slots k in order of the pair outputs
//             (+ the shared expert) (+ residual); NaN for a pair whose
//             expert index is out of range.
// No unit waits for another: the launches are ordered on the stream.
#include "common.h"
#include "decode_common.h"
#include "launch.h"

namespace moeq {

constexpr int kBThreads = 512;
constexpr int kBWaves = kBThreads / kWave;
constexpr int kBGRows = 16;   // gate/up rows per unit (two per wave)

// An empty asm that claims to modify v: the weights are reused for every
// token, and without it the compiler hoists their unpacked codes out of the
// token loop into (far too many) registers.
__device__ __forceinline__ void opaque(uint4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

// ---------------------------------------------------------------- gate / up
// LDS: [kBTok tokens][x interleaved (H floats)][kBTok][chunk sums (H/16)]
//      [bf16 scales/biases of the unit's gate and up rows]
template <int BITS, int CPL>
__global__ void __launch_bounds__(kBThreads) k_bgate(DecodeLayer L, BatchWs B, int M, int K,
                                                    const float* __restrict__ x) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  constexpr int kCpc = 128 / BITS;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int H = L.H;
  const int ngr = L.I / kBGRows;
  const int item = blockIdx.x;
  const bool shared = item >= B.max_tiles * ngr;
  int g, rows, e = 0, row0 = 0;
  if (!shared) {
    const int tile = item / ngr;
    g = item - tile * ngr;
    if (tile >= B.n_tiles[0]) return;
    const int4 T = B.tiles[tile];
    e = T.x;
    row0 = T.y;
    rows = T.z;
  } else {
    g = item - B.max_tiles * ngr;
    rows = M;
  }
  const QT Gq = shared ? L.sh_gate : L.gate;
  const QT Uq = shared ? L.sh_up : L.up;
  const int I = shared ? L.Is : L.I;
  const int nch = H / kCpc, wpr = H / (32 / BITS), gpr = H / kGroup, x16 = H / 4;
  const int i_base = g * kBGRows;
  const size_t erow = (size_t)e * I;
  __shared__ int s_tok[kBTok], s_pair[kBTok];
  // weights and scales first (clamped addresses, no branches), then x
  const int sb16 = kBGRows * gpr * 2 / 16;
  uint4 sbr;
  {
    const int qq = min(tid, 4 * sb16 - 1);
    const int q = qq / sb16, w = qq - q * sb16;
    const uint16_t* src = q == 0 ? Gq.scales : q == 1 ? Gq.biases : q == 2 ? Uq.scales : Uq.biases;
    sbr = reinterpret_cast<const uint4*>(src + (erow + i_base) * gpr)[w];
  }
  uint4 wg[2][CPL], wu[2][CPL];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const size_t row = erow + i_base + wid * 2 + rr;
    const uint4* g4 = reinterpret_cast<const uint4*>(Gq.q + row * wpr);
    const uint4* u4 = reinterpret_cast<const uint4*>(Uq.q + row * wpr);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = min(lane + kWave * j, nch - 1);
      wg[rr][j] = g4[c];
      wu[rr][j] = u4[c];
    }
  }
  float* xs = smem;                                    // [kBTok][H]
  float* xsum = xs + kBTok * H;                        // [kBTok][H/16]
  uint16_t* sbl = reinterpret_cast<uint16_t*>(xsum + kBTok * H / 16);
  if (tid < 4 * sb16) reinterpret_cast<uint4*>(sbl)[tid] = sbr;
  // the tile's tokens, kBTok at a time; the weights stay in registers
  for (int j0 = 0; j0 < rows; j0 += kBTok) {
  const int nj = min(kBTok, rows - j0);
  __syncthreads();                                     // the previous group is done with LDS
  if (tid < kBTok) {
    int tk = 0, pr = 0;
    if (tid < nj) {
      if (shared) {
        tk = j0 + tid;
      } else {
        pr = B.sorted[row0 + j0 + tid];
        tk = pr / K;
      }
    }
    s_tok[tid] = tk;
    s_pair[tid] = pr;
  }
  __syncthreads();
  for (int i = tid; i < nj * x16; i += kBThreads) {
    const int j = i / x16, f = i - j * x16;
    reinterpret_cast<float4*>(xs + j * H)[ilv<kCpc>(f, nch)] =
        reinterpret_cast<const float4*>(x + (size_t)s_tok[j] * H)[f];
  }
  __syncthreads();
  for (int j = 0; j < nj; ++j)
    chunk_sums<kCpc>(reinterpret_cast<const float4*>(xs + j * H), xsum + j * (H / 16), nch);
  __syncthreads();
  for (int j = 0; j < nj; ++j) {
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
      for (int c8 = 0; c8 < CPL; ++c8) {
        opaque(wg[rr][c8]);
        opaque(wu[rr][c8]);
      }
    const float4* x4 = reinterpret_cast<const float4*>(xs + j * H);
    const float* xsj = xsum + j * (H / 16);
    float pg[2], pu[2];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int i = wid * 2 + rr;
      float ag = 0.f, au = 0.f;
#pragma unroll
      for (int c8 = 0; c8 < CPL; ++c8) {
        const int c = lane + kWave * c8;
        if (c < nch) {
          const int grp = i * gpr + (c * kCpc) / kGroup;
          const float dg = chunk_dot<BITS>(wg[rr][c8], x4 + c, nch);
          const float du = chunk_dot<BITS>(wu[rr][c8], x4 + c, nch);
          ag = fmaf(bf16_to_f32(sbl[grp]), dg, fmaf(bf16_to_f32(sbl[kBGRows * gpr + grp]), xsj[c], ag));
          au = fmaf(bf16_to_f32(sbl[2 * kBGRows * gpr + grp]), du,
                    fmaf(bf16_to_f32(sbl[3 * kBGRows * gpr + grp]), xsj[c], au));
        }
      }
      pg[rr] = ag;
      pu[rr] = au;
    }
    const float gsum = treduce<2, 32>(pg, lane);
    const float usum = treduce<2, 32>(pu, lane);
    if ((lane & 31) == 0) {
      const int i = i_base + wid * 2 + tindex<2, 32>(lane);
      const float hv = silu(gsum) * usum;
      if (shared) B.hsh[(size_t)s_tok[j] * L.Is + i] = hv;
      else B.h[(size_t)s_pair[j] * L.I + i] = hv;
    }
  }
  if (shared && g == 0 && wid < nj) {
    // the shared_expert_gate logit of token s_tok[wid] (one row of H, its own bits)
    const int j = wid;
    const float* xsj = xs + j * H;
    const int eb = L.sh_eg.bits;
    const int cpce = 128 / eb;
    const int nche = H / cpce;
    float a = 0.f;
    for (int c = lane; c < nche; c += kWave) {
      const uint4 v = reinterpret_cast<const uint4*>(L.sh_eg.q)[c];
      const int gg = (c * cpce) / kGroup;
      float d = 0.f, xsm = 0.f;
      for (int q = 0; q < cpce; ++q) {
        const int col = c * cpce + q;
        const float xv = xsj[4 * ilv<kCpc>(col / 4, nch) + col % 4];
        const uint32_t word = q / (32 / eb) == 0 ? v.x : q / (32 / eb) == 1 ? v.y : q / (32 / eb) == 2 ? v.z : v.w;
        const uint32_t code = (word >> (eb * (q % (32 / eb)))) & ((1u << eb) - 1u);
        d = fmaf((float)code, xv, d);
        xsm += xv;
      }
      a = fmaf(bf16_to_f32(L.sh_eg.scales[gg]), d, fmaf(bf16_to_f32(L.sh_eg.biases[gg]), xsm, a));
    }
    a = wave_sum(a);
    if (lane == 0) B.sg[s_tok[j]] = a;
  }
  }
}

// ---------------------------------------------------------------------- down
// A wave holds 64/LPR rows, LPR lanes per row, NCL 16-byte chunks per lane.
// LDS: [kBTok][h interleaved (Imax floats)][kBTok][chunk sums]
template <int BITS, int LPR, int NCL>
__global__ void __launch_bounds__(kBThreads) k_bdown(DecodeLayer L, BatchWs B, int M, int K,
                                                    const float* __restrict__ wts) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  constexpr int kCpc = 128 / BITS;
  constexpr int kRpw = kWave / LPR;                    // rows per wave
  constexpr int kRows = kBWaves * kRpw;                // rows per unit
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int H = L.H;
  const int ndb = (H + kRows - 1) / kRows;
  const int item = blockIdx.x;
  const bool shared = item >= B.max_tiles * ndb;
  int cb, rows, e = 0, row0 = 0;
  if (!shared) {
    const int tile = item / ndb;
    cb = item - tile * ndb;
    if (tile >= B.n_tiles[0]) return;
    const int4 T = B.tiles[tile];
    e = T.x;
    row0 = T.y;
    rows = T.z;
  } else {
    cb = item - B.max_tiles * ndb;
    rows = M;
  }
  const QT Dq = shared ? L.sh_down : L.down;
  const int I = shared ? L.Is : L.I;
  const int cpr = I / kCpc;                            // chunks per down row
  const int gr = I / kGroup;
  const int r = cb * kRows + wid * kRpw + lane / LPR;  // the lane's output row
  const int rc = min(r, H - 1);
  const int ql = lane % LPR;
  const size_t drow = (size_t)e * H + rc;
  __shared__ int s_pair[kBTok], s_tok[kBTok];
  __shared__ float s_w[kBTok];
  // the lane's chunks, their scales and biases (clamped addresses, no branches)
  uint4 wv[NCL];
  float sc[NCL], bi[NCL];
#pragma unroll
  for (int j = 0; j < NCL; ++j) {
    const int q = min(ql + LPR * j, cpr - 1);
    wv[j] = reinterpret_cast<const uint4*>(Dq.q + drow * (I / (32 / BITS)))[q];
    const int grp = (q * kCpc) / kGroup;
    sc[j] = bf16_to_f32(Dq.scales[drow * gr + grp]);
    bi[j] = bf16_to_f32(Dq.biases[drow * gr + grp]);
  }
  float* hs = smem;                                    // [kBTok][I]
  float* hsum = hs + kBTok * I;                        // [kBTok][I/16]
  const int i4 = I / 4;
  // the tile's pairs, kBTok at a time; the weights stay in registers
  for (int j0 = 0; j0 < rows; j0 += kBTok) {
  const int nj = min(kBTok, rows - j0);
  __syncthreads();                                     // the previous group is done with LDS
  if (tid < kBTok) {
    int pr = 0, tk = 0;
    float wt = 0.f;
    if (tid < nj) {
      if (shared) {
        tk = j0 + tid;
        wt = 1.0f / (1.0f + __expf(-B.sg[tk]));
      } else {
        pr = B.sorted[row0 + j0 + tid];
        tk = pr / K;
        wt = wts[pr];
      }
    }
    s_pair[tid] = pr;
    s_tok[tid] = tk;
    s_w[tid] = wt;
  }
  __syncthreads();
  for (int i = tid; i < nj * i4; i += kBThreads) {
    const int j = i / i4, f = i - j * i4;
    const float* src = shared ? B.hsh + (size_t)s_tok[j] * L.Is : B.h + (size_t)s_pair[j] * L.I;
    reinterpret_cast<float4*>(hs + j * I)[ilv<kCpc>(f, cpr)] = reinterpret_cast<const float4*>(src)[f];
  }
  __syncthreads();
  for (int j = 0; j < nj; ++j)
    chunk_sums<kCpc>(reinterpret_cast<const float4*>(hs + j * I), hsum + j * (I / 16), cpr);
  __syncthreads();
  for (int j = 0; j < nj; ++j) {
#pragma unroll
    for (int c8 = 0; c8 < NCL; ++c8) opaque(wv[c8]);
    const float4* h4 = reinterpret_cast<const float4*>(hs + j * I);
    float acc = 0.f;
#pragma unroll
    for (int c8 = 0; c8 < NCL; ++c8) {
      const int q = ql + LPR * c8;
      if (q < cpr)
        acc = fmaf(sc[c8], chunk_dot<BITS>(wv[c8], h4 + q, cpr), fmaf(bi[c8], hsum[j * (I / 16) + q], acc));
    }
    float v[1] = {acc};
    const float tot = treduce<1, LPR / 2>(v, lane);
    if (ql == 0 && r < H) {
      if (shared) B.ysh[(size_t)s_tok[j] * H + r] = s_w[j] * tot;
      else B.ypair[(size_t)s_pair[j] * H + r] = s_w[j] * tot;
    }
  }
  }
}

// y[t][c] = sum over slots k in order of ypair[t*K+k][c] (+ shared) (+ residual);
// NaN where a slot's expert index is out of range
__global__ void __launch_bounds__(256) k_bcombine(const float* __restrict__ ypair,
                                                  const float* __restrict__ ysh,
                                                  const int32_t* __restrict__ idx,
                                                  const float* __restrict__ residual, int M, int K,
                                                  int H, int E, float* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // 4-column group
  if (i >= (int64_t)M * H / 4) return;
  const int64_t t = (i * 4) / H;
  const int64_t c = i * 4 - t * H;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = 0; k < K; ++k) {
    const int64_t p = t * K + k;
    const int e = idx[p];
    if (e >= 0 && e < E) {
      const float4 v = *reinterpret_cast<const float4*>(ypair + p * H + c);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    } else {
      s = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""));
    }
  }
  if (ysh) {
    const float4 v = *reinterpret_cast<const float4*>(ysh + t * H + c);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  if (residual) {
    const float4 v = *reinterpret_cast<const float4*>(residual + t * H + c);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  *reinterpret_cast<float4*>(y + t * H + c) = s;
}

// ---------------------------------------------------------------- host side
static int b_cpl(int H, int bits) {
  const int nch = H / (128 / bits);
  return nch <= kWave ? 1 : nch <= 2 * kWave ? 2 : nch <= 4 * kWave ? 4 : 0;
}

// lanes per down row (a power of two, 8..64) and chunks per lane
static void b_lpr(int I, int bits, int* lpr, int* ncl) {
  const int cpr = I / (128 / bits);
  int l = 8;
  while (l < cpr && l < kWave) l *= 2;
  *lpr = l;
  const int n = (cpr + l - 1) / l;
  *ncl = n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : 0;
}

bool batch_supported(const DecodeLayer& L) {
  const int b = L.gate.bits;
  if (L.H > 4096 || !b_cpl(L.H, b)) return false;
  if (4 * kBGRows * (L.H / kGroup) * 2 / 16 > kBThreads) return false;
  if (L.I % kBGRows) return false;
  int lpr, ncl;
  b_lpr(L.I, b, &lpr, &ncl);
  if (!ncl) return false;
  if (L.has_shared) {
    if (L.sh_gate.bits != b || L.Is % kBGRows) return false;
    int l2, n2;
    b_lpr(L.Is, b, &l2, &n2);
    if (l2 != lpr || n2 != ncl) return false;
    if (L.sh_eg.bits != 2 && L.sh_eg.bits != 4 && L.sh_eg.bits != 8) return false;
  }
  return true;
}

static size_t bgate_lds(const DecodeLayer& L) {
  return sizeof(float) * (size_t)kBTok * (L.H + L.H / 16) + 2 * 4 * kBGRows * (L.H / kGroup);
}
static size_t bdown_lds(const DecodeLayer& L) {
  const int Im = L.has_shared && L.Is > L.I ? L.Is : L.I;
  return sizeof(float) * (size_t)kBTok * (Im + Im / 16);
}

int launch_batch_forward(const DecodeLayer& L, const float* x, const int32_t* idx, const float* w,
                         int M, int K, const float* residual, float* y, const BatchWs& B,
                         hipStream_t s) {
  const int b = L.gate.bits;
  const int n = M * K;
  launch_sort_pairs_bm(idx, n, L.E, B.sort, kBTile, s);
  const int ngr = L.I / kBGRows;
  const int nst = L.has_shared ? 1 : 0;                // the shared expert: one tile of all M tokens
  const int ngs = L.has_shared ? L.Is / kBGRows : 0;
  const dim3 gg((unsigned)(B.max_tiles * ngr + nst * ngs));
  const size_t lg = bgate_lds(L);
  const int cpl = b_cpl(L.H, b);
// (dynamic LDS above 64 KB needs the kernel's limit raised first)
#define MOEQ_BG(B_, C_)                                                                     \
  if (b == B_ && cpl == C_) {                                                              \
    (void)hipFuncSetAttribute((const void*)k_bgate<B_, C_>,                                \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lg);         \
    hipLaunchKernelGGL((k_bgate<B_, C_>), gg, dim3(kBThreads), lg, s, L, B, M, K, x);      \
  }
  MOEQ_BG(8, 1) MOEQ_BG(8, 2) MOEQ_BG(8, 4) MOEQ_BG(4, 1) MOEQ_BG(4, 2) MOEQ_BG(4, 4)
  MOEQ_BG(2, 1) MOEQ_BG(2, 2) MOEQ_BG(2, 4)
#undef MOEQ_BG
  int lpr, ncl;
  b_lpr(L.I, b, &lpr, &ncl);
  const int rows_unit = kBWaves * (kWave / lpr);
  const int ndb = (L.H + rows_unit - 1) / rows_unit;
  const dim3 gd((unsigned)(B.max_tiles * ndb + nst * ndb));
  const size_t ld = bdown_lds(L);
#define MOEQ_BD(B_, L_, N_)                                                                 \
  if (b == B_ && lpr == L_ && ncl == N_) {                                                 \
    (void)hipFuncSetAttribute((const void*)k_bdown<B_, L_, N_>,                            \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)ld);         \
    hipLaunchKernelGGL((k_bdown<B_, L_, N_>), gd, dim3(kBThreads), ld, s, L, B, M, K, w);  \
  }
#define MOEQ_BD_B(B_) MOEQ_BD(B_, 8, 1) MOEQ_BD(B_, 16, 1) MOEQ_BD(B_, 32, 1) MOEQ_BD(B_, 64, 1) \
  MOEQ_BD(B_, 64, 2) MOEQ_BD(B_, 64, 4)
  MOEQ_BD_B(8) MOEQ_BD_B(4) MOEQ_BD_B(2)
#undef MOEQ_BD_B
#undef MOEQ_BD
  const int64_t total = (int64_t)M * L.H / 4;
  hipLaunchKernelGGL(k_bcombine, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, B.ypair,
                     L.has_shared ? B.ysh : nullptr, idx, residual, M, K, L.H, L.E, y);
  return 0;
}

}  // namespace moeq
