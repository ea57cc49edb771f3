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
// gather path, tiles of at most kBTile pairs), then
//   k_bgate   one unit = (tile, 64 gate/up rows): the tile's activations in
//             LDS, each wave streams 16 rows of gate and of up with the next
//             step's rows in flight, SwiGLU, h[pair]; the shared expert is
//             cut into tiles of kBTok tokens, and the units of its first rows
//             also compute the shared_expert_gate logits;
//   k_bdown   one unit = (tile, a slab of output rows): the same streaming
//             over down rows, scaled by the routing weight (or the sigmoid of
//             the shared gate) into a per-pair output row;
//   k_bcombine y[t] = sum over slots k in order of the pair outputs
//             (+ the shared expert) (+ residual); NaN for a pair whose
//             expert index is out of range.
// No unit waits for another: the launches are ordered on the stream.
#include "common.h"
#include "decode_common.h"
#include "launch.h"

namespace moeq {

constexpr int kBThreads = 256;               // four waves
constexpr int kBWaves = kBThreads / kWave;
constexpr int kBSlab = 64;                   // gate/up rows of a unit (16 per wave)
constexpr int kBDSteps = 8;                  // down: steps per wave
constexpr int kBRpl = 2;                     // down: rows per lane and step

// ---- byte-wise unpacking ----------------------------------------------------
// A 32-bit word of codes is split into passes whose four bytes each hold one
// code, converted with one byte-to-float instruction apiece:
//   2 bits: pass m = (w >> 2m) & 0x03030303, byte b = code 4b + m of the word
//   4 bits: pass m = (w >> 4m) & 0x0F0F0F0F, byte b = code 2b + m
//   8 bits: the word itself, byte b = code b
// (the empty asm hides the mask from the compiler, which would otherwise
// fold it into one bit-field extract per code)
template <int BITS>
__device__ __forceinline__ uint32_t upass(uint32_t w, int m) {
  uint32_t t = w;
  if constexpr (BITS == 2) t = (w >> (2 * m)) & 0x03030303u;
  else if constexpr (BITS == 4) t = (w >> (4 * m)) & 0x0F0F0F0Fu;
  asm volatile("" : "+v"(t));
  return t;
}

__device__ __forceinline__ float comp(const float4& v, int c) {
  return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}

// d[r][t] += (codes of the 16-byte chunk v[r]) . (activations of token t).
// x4 points at float4 0 of the lane's chunk of token 0 in the chunk-interleaved
// layout (float4 f at x4[f * stride], token t at + t * tstride).  Every code is
// converted once and used for all T tokens.
template <int BITS, int R, int T>
__device__ __forceinline__ void chunk_dots(const uint4 (&v)[R], const float4* x4, int stride,
                                           int tstride, float (&d)[R][T]) {
  constexpr int kPasses = BITS == 2 ? 4 : BITS == 4 ? 2 : 1;
  constexpr int kF = 8 / BITS;                 // float4s of activations per word
#pragma unroll
  for (int wi = 0; wi < 4; ++wi) {
    float4 xv[T][kF];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int f = 0; f < kF; ++f) xv[t][f] = x4[t * tstride + (wi * kF + f) * stride];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t w = wi == 0 ? v[r].x : wi == 1 ? v[r].y : wi == 2 ? v[r].z : v[r].w;
#pragma unroll
      for (int m = 0; m < kPasses; ++m) {
        const uint32_t tb = upass<BITS>(w, m);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float c = (float)((tb >> (8 * b)) & 0xFFu);
          // the code's place among the word's activations
          const int f = BITS == 2 ? b : BITS == 4 ? b / 2 : 0;
          const int cc = BITS == 2 ? m : BITS == 4 ? 2 * (b % 2) + m : b;
#pragma unroll
          for (int t = 0; t < T; ++t) d[r][t] = fmaf(c, comp(xv[t][f], cc), d[r][t]);
        }
      }
      // one row of one word at a time: the compiler would otherwise convert
      // (and fetch activations for) every word of every row at once and run
      // out of registers
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// stage nt activation rows (H floats each, row t at src[t]) chunk-interleaved
// into LDS with their chunk sums
template <int CPC>
__device__ __forceinline__ void stage_rows(float* xs, float* xsum, const float* const* src, int nt,
                                           int H) {
  const int nch = H / CPC, x16 = H / 4;
  for (int i = threadIdx.x; i < nt * x16; i += kBThreads) {
    const int j = i / x16, f = i - j * x16;
    reinterpret_cast<float4*>(xs + j * H)[ilv<CPC>(f, nch)] = reinterpret_cast<const float4*>(src[j])[f];
  }
  __syncthreads();
  for (int j = 0; j < nt; ++j)
    chunk_sums<CPC>(reinterpret_cast<const float4*>(xs + j * H), xsum + j * (H / 16), nch);
  __syncthreads();
}

// ---------------------------------------------------------------- gate / up
// One unit = (tile of at most kBTok pairs, or kBTok tokens of the shared
// expert) x (kBSlab rows of gate and of up).  A wave streams its 16 rows RPS
// at a time, the next step's rows (and their scales and biases) in flight
// while the current ones are applied to the tile's tokens.
// LDS: [kBTok][x interleaved (H floats)][kBTok][chunk sums (H/16)]
template <int BITS, int CPL, int RPS>
struct GateStep {
  uint4 g[RPS][CPL], u[RPS][CPL];
  uint32_t gs[RPS][CPL], gb[RPS][CPL], us[RPS][CPL], ub[RPS][CPL];
};

template <int BITS, int CPL, int RPS>
__device__ __forceinline__ void gate_load(GateStep<BITS, CPL, RPS>& S, const QT& Gq, const QT& Uq,
                                          size_t row, int lane, int nch, int wpr, int gpr) {
  constexpr int kCpc = 128 / BITS;
#pragma unroll
  for (int rr = 0; rr < RPS; ++rr) {
    const size_t rw = row + rr;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = min(lane + kWave * j, nch - 1);
      const int grp = group_of(c * kCpc, Gq.group_size);
      S.g[rr][j] = reinterpret_cast<const uint4*>(Gq.q + rw * wpr)[c];
      S.u[rr][j] = reinterpret_cast<const uint4*>(Uq.q + rw * wpr)[c];
      S.gs[rr][j] = Gq.scales[rw * gpr + grp];
      S.gb[rr][j] = Gq.biases[rw * gpr + grp];
      S.us[rr][j] = Uq.scales[rw * gpr + grp];
      S.ub[rr][j] = Uq.biases[rw * gpr + grp];
    }
  }
}

template <int BITS, int CPL, int RPS, int T>
__device__ __forceinline__ void gate_rows(const DecodeLayer& L, const BatchWs& B, const QT& Gq,
                                          const QT& Uq, size_t erow, int i0, bool shared,
                                          const float* xs, const float* xsum, const int* s_tok,
                                          const int* s_pair, int nt, int lane) {
  constexpr int kCpc = 128 / BITS;
  constexpr int kSteps = kBSlab / kBWaves / RPS;
  constexpr int kN = RPS * T;
  const int H = L.H;
  const int nch = H / kCpc, wpr = H / (32 / BITS), gpr = H >> __builtin_ctz((unsigned)Gq.group_size);
  GateStep<BITS, CPL, RPS> cur, nxt;
  gate_load<BITS, CPL, RPS>(cur, Gq, Uq, erow + i0, lane, nch, wpr, gpr);
#pragma unroll 1
  for (int s = 0; s < kSteps; ++s) {
    if (s + 1 < kSteps) gate_load<BITS, CPL, RPS>(nxt, Gq, Uq, erow + i0 + (s + 1) * RPS, lane, nch, wpr, gpr);
    float ag[RPS][T], au[RPS][T];
#pragma unroll
    for (int rr = 0; rr < RPS; ++rr)
#pragma unroll
      for (int t = 0; t < T; ++t) ag[rr][t] = au[rr][t] = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c0 = lane + kWave * j;
      const bool ok = c0 < nch;
      const int c = min(c0, nch - 1);
      uint4 v[2 * RPS];
#pragma unroll
      for (int rr = 0; rr < RPS; ++rr) {
        v[rr] = cur.g[rr][j];
        v[RPS + rr] = cur.u[rr][j];
      }
      float d[2 * RPS][T];
#pragma unroll
      for (int r = 0; r < 2 * RPS; ++r)
#pragma unroll
        for (int t = 0; t < T; ++t) d[r][t] = 0.f;
      chunk_dots<BITS, 2 * RPS, T>(v, reinterpret_cast<const float4*>(xs) + c, nch, H / 4, d);
#pragma unroll
      for (int rr = 0; rr < RPS; ++rr) {
        const float gsc = ok ? bf16_to_f32(cur.gs[rr][j]) : 0.f, gbi = ok ? bf16_to_f32(cur.gb[rr][j]) : 0.f;
        const float usc = ok ? bf16_to_f32(cur.us[rr][j]) : 0.f, ubi = ok ? bf16_to_f32(cur.ub[rr][j]) : 0.f;
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const float sm = xsum[t * (H / 16) + c];
          ag[rr][t] = fmaf(gsc, d[rr][t], fmaf(gbi, sm, ag[rr][t]));
          au[rr][t] = fmaf(usc, d[RPS + rr][t], fmaf(ubi, sm, au[rr][t]));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    float pg[kN], pu[kN];
#pragma unroll
    for (int rr = 0; rr < RPS; ++rr)
#pragma unroll
      for (int t = 0; t < T; ++t) {
        pg[rr * T + t] = ag[rr][t];
        pu[rr * T + t] = au[rr][t];
      }
    const float gsum = treduce<kN, 32>(pg, lane);
    const float usum = treduce<kN, 32>(pu, lane);
    const int vi = tindex<kN, 32>(lane);
    const int rr = vi / T, t = vi - rr * T;
    if ((lane & (kWave / kN - 1)) == 0 && t < nt) {
      const int i = i0 + s * RPS + rr;
      const float hv = silu(gsum) * usum;
      if (shared) B.hsh[(size_t)s_tok[t] * L.Is + i] = hv;
      else B.h[(size_t)s_pair[t] * L.I + i] = hv;
    }
    if (s + 1 < kSteps) cur = nxt;
  }
}

template <int BITS, int CPL, int RPS>
__global__ void __launch_bounds__(kBThreads) __attribute__((amdgpu_waves_per_eu(3)))
k_bgate(DecodeLayer L, BatchWs B, int M, int K, const float* __restrict__ x) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  constexpr int kCpc = 128 / BITS;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);   // uniform: row addresses in SGPRs
  const int H = L.H;
  const int nsl = L.I / kBSlab;
  const int item = blockIdx.x;
  const bool shared = item >= B.max_tiles * nsl;
  int sl, nt, e = 0, row0 = 0, tg = 0;
  if (!shared) {
    const int tile = item / nsl;
    sl = item - tile * nsl;
    if (tile >= B.n_tiles[0]) return;
    const int4 T = B.tiles[tile];
    e = T.x;
    row0 = T.y;
    nt = T.z;
  } else {
    const int nss = L.Is / kBSlab;
    const int it = item - B.max_tiles * nsl;
    tg = it / nss;
    sl = it - tg * nss;
    nt = min(kBTok, M - tg * kBTok);
  }
  const QT Gq = shared ? L.sh_gate : L.gate;
  const QT Uq = shared ? L.sh_up : L.up;
  const int I = shared ? L.Is : L.I;
  const size_t erow = (size_t)e * I;
  const int i0 = sl * kBSlab + wid * (kBSlab / kBWaves);
  // the units of the shared expert's first rows also compute their tokens'
  // shared_expert_gate logits (one row of H, its own bits): one 16-byte chunk
  // per thread (H * bits / 128 <= kBThreads), loaded up front
  const bool sgu = shared && sl == 0;               // uniform over the block
  const int eb = L.sh_eg.bits, cpce = 128 / eb, nche = H / cpce;
  uint4 egv = make_uint4(0u, 0u, 0u, 0u);
  uint32_t egsb = 0u;
  if (sgu) {
    const int c = min(tid, nche - 1);
    const int gg = group_of(c * cpce, L.sh_eg.group_size);
    egv = reinterpret_cast<const uint4*>(L.sh_eg.q)[c];
    egsb = (uint32_t)L.sh_eg.scales[gg] | ((uint32_t)L.sh_eg.biases[gg] << 16);
  }
  __shared__ int s_tok[kBTok], s_pair[kBTok];
  __shared__ const float* s_src[kBTok];
  if (tid < kBTok) {
    int tk = 0, pr = 0;
    if (tid < nt) {
      if (shared) {
        tk = tg * kBTok + tid;
      } else {
        pr = B.sorted[row0 + tid];
        tk = pr / K;
      }
    }
    s_tok[tid] = tk;
    s_pair[tid] = pr;
    s_src[tid] = x + (size_t)tk * H;
  }
  __syncthreads();
  float* xs = smem;                                    // [kBTok][H]
  float* xsum = xs + kBTok * H;                        // [kBTok][H/16]
  stage_rows<kCpc>(xs, xsum, s_src, nt, H);
  // (the gate row's chunk waits in LDS, not in registers, while the rows stream)
  __shared__ uint4 s_egv[kBThreads];
  __shared__ uint32_t s_egsb[kBThreads];
  if (sgu) {
    s_egv[tid] = egv;
    s_egsb[tid] = egsb;
  }
  if (nt == 1) gate_rows<BITS, CPL, RPS, 1>(L, B, Gq, Uq, erow, i0, shared, xs, xsum, s_tok, s_pair, nt, lane);
  else gate_rows<BITS, CPL, RPS, kBTok>(L, B, Gq, Uq, erow, i0, shared, xs, xsum, s_tok, s_pair, nt, lane);
  if (sgu) {
    // each thread's chunk for every token of the tile, then the block's sums
    // in wave order
    __shared__ float sgp[kBWaves][kBTok];
    const int nch = H / kCpc;
    float a[kBTok];
#pragma unroll
    for (int j = 0; j < kBTok; ++j) {
      a[j] = 0.f;
      if (tid < nche && j < nt) {
        const uint4 egv = s_egv[tid];
        const uint32_t egsb = s_egsb[tid];
        const float* xsj = xs + j * H;
        float d = 0.f, xsm = 0.f;
        for (int q = 0; q < cpce; ++q) {
          const int col = tid * cpce + q;
          const float xv = xsj[4 * ilv<kCpc>(col / 4, nch) + col % 4];
          const uint32_t word = q / (32 / eb) == 0 ? egv.x : q / (32 / eb) == 1 ? egv.y : q / (32 / eb) == 2 ? egv.z : egv.w;
          const uint32_t code = (word >> (eb * (q % (32 / eb)))) & ((1u << eb) - 1u);
          d = fmaf((float)code, xv, d);
          xsm += xv;
        }
        a[j] = fmaf(bf16_to_f32(egsb & 0xFFFFu), d, bf16_to_f32(egsb >> 16) * xsm);
      }
      a[j] = wave_sum(a[j]);
      if (lane == 0) sgp[wid][j] = a[j];
    }
    __syncthreads();
    if (tid < nt) {
      float tot = 0.f;
      for (int w = 0; w < kBWaves; ++w) tot += sgp[w][tid];
      B.sg[s_tok[tid]] = tot;
    }
  }
}

// ---------------------------------------------------------------------- down
// One unit = (tile or kBTok shared tokens) x (kBWaves * kBDSteps * kBRpl *
// 64/LPR output rows).  LPR lanes share a row, NCL 16-byte chunks per lane;
// a lane takes kBRpl rows per step, the next step's in flight.
// LDS: [kBTok][h interleaved (Imax floats)][kBTok][chunk sums]
template <int BITS, int NCL>
struct DownStep {
  uint4 w[kBRpl][NCL];
  uint32_t sc[kBRpl][NCL], bi[kBRpl][NCL];
};

template <int BITS, int LPR, int NCL>
__device__ __forceinline__ void down_load(DownStep<BITS, NCL>& S, const QT& Dq, size_t erow, int r,
                                          int H, int I, int ql) {
  constexpr int kCpc = 128 / BITS;
  constexpr int kGrp = kWave / LPR;
  const int cpr = I / kCpc, gr = I >> __builtin_ctz((unsigned)Dq.group_size), wpr = I / (32 / BITS);
#pragma unroll
  for (int rr = 0; rr < kBRpl; ++rr) {
    const size_t row = erow + min(r + rr * kGrp, H - 1);
#pragma unroll
    for (int j = 0; j < NCL; ++j) {
      const int q = min(ql + LPR * j, cpr - 1);
      const int grp = group_of(q * kCpc, Dq.group_size);
      S.w[rr][j] = reinterpret_cast<const uint4*>(Dq.q + row * wpr)[q];
      S.sc[rr][j] = Dq.scales[row * gr + grp];
      S.bi[rr][j] = Dq.biases[row * gr + grp];
    }
  }
}

template <int BITS, int LPR, int NCL, int T>
__device__ __forceinline__ void down_rows(const DecodeLayer& L, const BatchWs& B, const QT& Dq,
                                          size_t erow, int rbase, bool shared, const float* hs,
                                          const float* hsum, const int* s_tok, const int* s_pair,
                                          const float* s_w, int nt, int lane) {
  constexpr int kCpc = 128 / BITS;
  constexpr int kGrp = kWave / LPR;
  constexpr int kRowsStep = kBRpl * kGrp;
  constexpr int kN = kBRpl * T;
  const int H = L.H;
  const int I = shared ? L.Is : L.I;
  const int cpr = I / kCpc;
  const int ql = lane % LPR;
  const int rl = lane / LPR;
  DownStep<BITS, NCL> cur, nxt;
  down_load<BITS, LPR, NCL>(cur, Dq, erow, rbase + rl, H, I, ql);
#pragma unroll 1
  for (int s = 0; s < kBDSteps; ++s) {
    if (s + 1 < kBDSteps) down_load<BITS, LPR, NCL>(nxt, Dq, erow, rbase + (s + 1) * kRowsStep + rl, H, I, ql);
    float acc[kBRpl][T];
#pragma unroll
    for (int rr = 0; rr < kBRpl; ++rr)
#pragma unroll
      for (int t = 0; t < T; ++t) acc[rr][t] = 0.f;
#pragma unroll
    for (int j = 0; j < NCL; ++j) {
      const int q0 = ql + LPR * j;
      const bool ok = q0 < cpr;
      const int q = min(q0, cpr - 1);
      uint4 v[kBRpl];
#pragma unroll
      for (int rr = 0; rr < kBRpl; ++rr) v[rr] = cur.w[rr][j];
      float d[kBRpl][T];
#pragma unroll
      for (int rr = 0; rr < kBRpl; ++rr)
#pragma unroll
        for (int t = 0; t < T; ++t) d[rr][t] = 0.f;
      chunk_dots<BITS, kBRpl, T>(v, reinterpret_cast<const float4*>(hs) + q, cpr, I / 4, d);
#pragma unroll
      for (int rr = 0; rr < kBRpl; ++rr) {
        const float sc = ok ? bf16_to_f32(cur.sc[rr][j]) : 0.f, bi = ok ? bf16_to_f32(cur.bi[rr][j]) : 0.f;
#pragma unroll
        for (int t = 0; t < T; ++t)
          acc[rr][t] = fmaf(sc, d[rr][t], fmaf(bi, hsum[t * (I / 16) + q], acc[rr][t]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    float pv[kN];
#pragma unroll
    for (int rr = 0; rr < kBRpl; ++rr)
#pragma unroll
      for (int t = 0; t < T; ++t) pv[rr * T + t] = acc[rr][t];
    const float tot = treduce<kN, LPR / 2>(pv, lane);
    const int vi = tindex<kN, LPR / 2>(lane);
    const int rr = vi / T, t = vi - rr * T;
    const int r = rbase + s * kRowsStep + rr * kGrp + rl;
    if ((ql & (LPR / kN - 1)) == 0 && t < nt && r < H) {
      if (shared) B.ysh[(size_t)s_tok[t] * H + r] = s_w[t] * tot;
      else B.ypair[(size_t)s_pair[t] * H + r] = s_w[t] * tot;
    }
    if (s + 1 < kBDSteps) cur = nxt;
  }
}

template <int BITS, int LPR, int NCL>
__global__ void __launch_bounds__(kBThreads) __attribute__((amdgpu_waves_per_eu(3)))
k_bdown(DecodeLayer L, BatchWs B, int M, int K, const float* __restrict__ wts) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  constexpr int kCpc = 128 / BITS;
  constexpr int kRowsStep = kBRpl * (kWave / LPR);
  constexpr int kRowsUnit = kBWaves * kBDSteps * kRowsStep;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);   // uniform: row addresses in SGPRs
  const int H = L.H;
  const int ndb = (H + kRowsUnit - 1) / kRowsUnit;
  const int item = blockIdx.x;
  const bool shared = item >= B.max_tiles * ndb;
  int cb, nt, e = 0, row0 = 0, tg = 0;
  if (!shared) {
    const int tile = item / ndb;
    cb = item - tile * ndb;
    if (tile >= B.n_tiles[0]) return;
    const int4 T = B.tiles[tile];
    e = T.x;
    row0 = T.y;
    nt = T.z;
  } else {
    const int it = item - B.max_tiles * ndb;
    tg = it / ndb;
    cb = it - tg * ndb;
    nt = min(kBTok, M - tg * kBTok);
  }
  const QT Dq = shared ? L.sh_down : L.down;
  const int I = shared ? L.Is : L.I;
  __shared__ int s_pair[kBTok], s_tok[kBTok];
  __shared__ float s_w[kBTok];
  __shared__ const float* s_src[kBTok];
  if (tid < kBTok) {
    int pr = 0, tk = 0;
    float wt = 0.f;
    if (tid < nt) {
      if (shared) {
        tk = tg * kBTok + tid;
        wt = 1.0f / (1.0f + __expf(-B.sg[tk]));
      } else {
        pr = B.sorted[row0 + tid];
        tk = pr / K;
        wt = wts[pr];
      }
    }
    s_pair[tid] = pr;
    s_tok[tid] = tk;
    s_w[tid] = wt;
    s_src[tid] = shared ? B.hsh + (size_t)tk * L.Is : B.h + (size_t)pr * L.I;
  }
  __syncthreads();
  float* hs = smem;                                    // [kBTok][I]
  float* hsum = hs + kBTok * I;                        // [kBTok][I/16]
  stage_rows<kCpc>(hs, hsum, s_src, nt, I);
  const int rbase = cb * kRowsUnit + wid * kBDSteps * kRowsStep;
  const size_t erow = (size_t)e * H;
  if (nt == 1) down_rows<BITS, LPR, NCL, 1>(L, B, Dq, erow, rbase, shared, hs, hsum, s_tok, s_pair, s_w, nt, lane);
  else down_rows<BITS, LPR, NCL, kBTok>(L, B, Dq, erow, rbase, shared, hs, hsum, s_tok, s_pair, s_w, nt, lane);
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
  if (L.I % kBSlab) return false;
  int lpr, ncl;
  b_lpr(L.I, b, &lpr, &ncl);
  if (!ncl) return false;
  if (L.has_shared) {
    if (L.sh_gate.bits != b || L.Is % kBSlab) return false;
    int l2, n2;
    b_lpr(L.Is, b, &l2, &n2);
    if (l2 != lpr || n2 != ncl) return false;
    if (L.sh_eg.bits != 2 && L.sh_eg.bits != 4 && L.sh_eg.bits != 8) return false;
  }
  return true;
}

static size_t bgate_lds(const DecodeLayer& L) {
  return sizeof(float) * (size_t)kBTok * (L.H + L.H / 16);
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
  const int ntg = L.has_shared ? (M + kBTok - 1) / kBTok : 0;   // shared-expert token groups
  const int nsl = L.I / kBSlab, nss = L.has_shared ? L.Is / kBSlab : 0;
  const dim3 gg((unsigned)(B.max_tiles * nsl + ntg * nss));
  const size_t lg = bgate_lds(L);
  const int cpl = b_cpl(L.H, b);
#define MOEQ_BG(B_, C_, R_)                                                                   \
  if (b == B_ && cpl == C_) {                                                                \
    MOEQ_ALLOW_FULL_LDS((k_bgate<B_, C_, R_>), lg);                                            \
    hipLaunchKernelGGL((k_bgate<B_, C_, R_>), gg, dim3(kBThreads), lg, s, L, B, M, K, x);    \
  }
  MOEQ_BG(8, 1, 2) MOEQ_BG(8, 2, 1) MOEQ_BG(8, 4, 1) MOEQ_BG(4, 1, 2) MOEQ_BG(4, 2, 1)
  MOEQ_BG(4, 4, 1) MOEQ_BG(2, 1, 2) MOEQ_BG(2, 2, 1) MOEQ_BG(2, 4, 1)
#undef MOEQ_BG
  int lpr, ncl;
  b_lpr(L.I, b, &lpr, &ncl);
  const int rows_unit = kBWaves * kBDSteps * kBRpl * (kWave / lpr);
  const int ndb = (L.H + rows_unit - 1) / rows_unit;
  const dim3 gd((unsigned)(B.max_tiles * ndb + ntg * ndb));
  const size_t ld = bdown_lds(L);
#define MOEQ_BD(B_, L_, N_)                                                                 \
  if (b == B_ && lpr == L_ && ncl == N_) {                                                 \
    MOEQ_ALLOW_FULL_LDS((k_bdown<B_, L_, N_>), ld);                                            \
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
