// Decode expert forward (fp32 activations, small M) as ONE launch.
//
// The step per selected expert (markbaseengine MOE_ROUTER_WORKS_BREAKTHROUGH,
// "Forward Pass Sequence": expertFusedGateUp, expertDown, accumulateResults;
// flash-moe-inference kernels swiglu and moe_combine_residual):
//   h_k = silu(Gate_e x) * (Up_e x),   y = sum_k w_k Down_e h_k
//         (+ sigmoid(sg . x) * FFN_shared(x)) (+ residual).
//
// Work units by block index (G units first, then D units):
//   G units  (pair p = token*S + slot, 16 intermediate rows): gate and up rows
//            of the pair's expert against x, SwiGLU, h[p][i]; the first G unit
//            of a shared-expert pair also computes the shared_expert_gate
//            logit.  Each G unit counts its arrival for token t; the one that
//            completes the count raises ready[t].
//   D units  (token t, 8 output rows): issue the weight loads of their rows
//            for all S slots at once, wait for ready[t], stage h of all S
//            pairs in LDS and produce whole output rows,
//            y = sum_k w_k Down_k h_k (+ sigmoid(sg) Down_sh h_sh) (+ residual),
//            with one fixed reduction order, so results are bitwise
//            reproducible and no data crosses blocks twice.  The last D unit of
//            a token to arrive lowers ready[t] for the next launch.
// Workgroups are dispatched in index order within each XCD, so when a D unit
// runs, every G unit of its XCD has been dispatched, and G units never wait:
// each wait ends.  Waits are bounded anyway: one that exceeds its spin limit
// records an error word in the workspace and gives up instead of hanging.
// Arrivals are counted with two-level counters (see arrive()).
//
// Latency is what bounds a decode layer, so every unit issues all of its HBM
// loads (weight rows, and the rows' bf16 scales and biases, staged through
// LDS) before it touches any result, and units are sized so that a whole
// layer's blocks are resident at once.  Rows are streamed in 16-byte chunks
// (128/BITS codes, never straddling a 64-column group); a chunk contributes
// s*(sum_j q_j a_j) + b*(sum_j a_j) with the activation's chunk sums
// precomputed once per block in LDS.
#include "common.h"
#include "launch.h"

namespace moeq {

constexpr int kGRows = 16;    // intermediate rows per G unit (four per wave)
constexpr int kDRows = 8;     // output rows per D unit (two per wave)
constexpr int kSpinLimit = 1 << 26;
constexpr int kLine = kLineInts;
constexpr int kCtrLines = 2 * (1 + kFan) + 1;   // per token: G counter, D counter, ready

// ---- coherent (agent-scope) loads/stores for data crossing blocks ----------
__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_coh64(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Data that crosses blocks is written and read only with agent-scope (sc1)
// accesses, which are coherent across the XCDs' L2s, so publishing needs no
// cache maintenance: drain this wave's outstanding memory operations before
// the counter update that announces them.
__device__ __forceinline__ void drain() { __builtin_amdgcn_s_waitcnt(0); }

// wait (one thread) until *flag != 0; returns false if the spin limit hit
__device__ __forceinline__ bool wait_flag(int* flag) {
  for (int i = 0; i < kSpinLimit; ++i) {
    if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return true;
    __builtin_amdgcn_s_sleep(4);
  }
  return false;
}

// Activations live in LDS chunk-interleaved: float4 number f of chunk c sits at
// a4[f * stride + c], so lanes working on consecutive chunks read consecutive
// 16-byte words (a plain [c][f] layout puts them 16*BITS bytes apart and every
// read becomes a many-way bank conflict).
//
// dot of one 16-byte chunk of BITS-bit codes with its activations
template <int BITS>
__device__ __forceinline__ float chunk_dot(const uint4& v, const float4* a4, int stride) {
  constexpr int kCpc = 128 / BITS;
  float d = 0.f;
#pragma unroll
  for (int j = 0; j < kCpc; j += 4) {
    const float4 av = a4[(j / 4) * stride];
    d = fmaf((float)chunk_code<BITS>(v, j + 0), av.x, d);
    d = fmaf((float)chunk_code<BITS>(v, j + 1), av.y, d);
    d = fmaf((float)chunk_code<BITS>(v, j + 2), av.z, d);
    d = fmaf((float)chunk_code<BITS>(v, j + 3), av.w, d);
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

// LDS of a block: [activation][its chunk sums (n/16 floats max)][the unit's
// bf16 scales and biases]
template <int BITS, int CPL, int DCH>
__global__ void __launch_bounds__(256) k_dec_fused(DecodeLayer L, DecPlan P,
                                                   const float* __restrict__ x,
                                                   const int32_t* __restrict__ idx,
                                                   const float* __restrict__ wts,
                                                   const float* __restrict__ residual,
                                                   float* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ int s_last;
  constexpr int kCpc = 128 / BITS;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  // counter lines: [0] error word, then per token kCtrLines lines: the G
  // arrival counter, the D arrival counter and the ready flag
  int* err = P.ctr;
  auto tok_lines = [&](int tt) { return P.ctr + (size_t)kLine * (1 + (size_t)tt * kCtrLines); };
  const int u = blockIdx.x;
  const int S = P.S, K = P.K, H = L.H;

  if (u < P.g_units) {
    // ------------------------------------------------------------ G unit
    const int upt = K * P.ng_routed + (L.has_shared ? P.ng_shared : 0);
    const int t = u / upt;
    const int r = u - t * upt;
    const bool shared = r >= K * P.ng_routed;
    const int k = shared ? K : r / P.ng_routed;
    const int g = shared ? r - K * P.ng_routed : r - k * P.ng_routed;
    const int p = t * S + k;
    const int I = shared ? L.Is : L.I;
    const QT& Gq = shared ? L.sh_gate : L.gate;
    const QT& Uq = shared ? L.sh_up : L.up;
    bool valid = true;
    size_t erow = 0;                                  // first row of the expert
    if (!shared) {
      const int e = idx[(size_t)t * K + k];
      valid = e >= 0 && e < L.E;
      erow = (size_t)(valid ? e : 0) * L.I;
    }
    const int i_base = g * kGRows;                    // the unit's first row
    const int nrows = min(kGRows, I - i_base);
    const int nch = H / kCpc;                         // chunks per row
    const int wpr = H / (32 / BITS);                  // words per row
    const int gpr = H / kGroup;                       // groups per row
    // 1) issue every HBM load, first what is needed first: x and the unit's
    //    scales/biases (contiguous: rows x groups bf16), then 4 rows x (gate,
    //    up) per wave
    const int x16 = H / 4;
    uint4 xr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + j * 256;
      xr[j] = i < x16 ? reinterpret_cast<const uint4*>(x + (size_t)t * H)[i] : make_uint4(0, 0, 0, 0);
    }
    const int sb16 = nrows * gpr * 2 / 16;            // 16-byte words per tensor
    uint4 sbr[4];
    {
      const size_t o = (erow + i_base) * gpr;
      const uint4* src[4] = {reinterpret_cast<const uint4*>(Gq.scales + o),
                             reinterpret_cast<const uint4*>(Gq.biases + o),
                             reinterpret_cast<const uint4*>(Uq.scales + o),
                             reinterpret_cast<const uint4*>(Uq.biases + o)};
#pragma unroll
      for (int q = 0; q < 4; ++q) sbr[q] = tid < sb16 ? src[q][tid] : make_uint4(0, 0, 0, 0);
    }
    uint4 wg[4][CPL], wu[4][CPL];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int i = wid * 4 + rr;
      const size_t row = erow + i_base + (i < nrows ? i : 0);
      const uint4* g4 = reinterpret_cast<const uint4*>(Gq.q + row * wpr);
      const uint4* u4 = reinterpret_cast<const uint4*>(Uq.q + row * wpr);
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = lane + kWave * j;
        const bool ok = i < nrows && c < nch;
        wg[rr][j] = ok ? g4[c] : make_uint4(0, 0, 0, 0);
        wu[rr][j] = ok ? u4[c] : make_uint4(0, 0, 0, 0);
      }
    }
    // 2) stage x, its chunk sums and the scales/biases in LDS
    float* xs = smem;
    float* xsum = xs + H;
    uint16_t* sbl = reinterpret_cast<uint16_t*>(xsum + H / 16);   // [4][kGRows*gpr]
    float4* x4 = reinterpret_cast<float4*>(xs);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + j * 256;
      if (i < x16) x4[ilv<kCpc>(i, nch)] = reinterpret_cast<const float4&>(xr[j]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (tid < sb16) reinterpret_cast<uint4*>(sbl + q * kGRows * gpr)[tid] = sbr[q];
    __syncthreads();
    chunk_sums<kCpc>(x4, xsum, nch);
    __syncthreads();
    // 3) the wave's four rows: per-lane partials, then one transposed reduction
    float pg[4], pu[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int i = wid * 4 + rr;
      float ag = 0.f, au = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = lane + kWave * j;
        if (c < nch) {
          const int grp = i * gpr + (c * kCpc) / kGroup;
          const float dg = chunk_dot<BITS>(wg[rr][j], x4 + c, nch);
          const float du = chunk_dot<BITS>(wu[rr][j], x4 + c, nch);
          ag = fmaf(bf16_to_f32(sbl[grp]), dg, fmaf(bf16_to_f32(sbl[kGRows * gpr + grp]), xsum[c], ag));
          au = fmaf(bf16_to_f32(sbl[2 * kGRows * gpr + grp]), du,
                    fmaf(bf16_to_f32(sbl[3 * kGRows * gpr + grp]), xsum[c], au));
        }
      }
      pg[rr] = ag;
      pu[rr] = au;
    }
    const float gsum = treduce<4, 32>(pg, lane);
    const float usum = treduce<4, 32>(pu, lane);
    if ((lane & 15) == 0) {
      const int i = wid * 4 + tindex<4, 32>(lane);
      if (i < nrows)
        st_coh(P.h + (size_t)p * P.Imax + i_base + i, valid ? silu(gsum) * usum : __builtin_nanf(""));
    }
    if (shared && g == 0 && wid == 0) {
      // the shared_expert_gate logit of token t (one row of H, its own bits)
      const int eb = L.sh_eg.bits;
      const int cpce = 128 / eb;
      const int nche = H / cpce;
      float a = 0.f;
      for (int c = lane; c < nche; c += kWave) {
        const uint4 v = reinterpret_cast<const uint4*>(L.sh_eg.q)[c];
        const int gg = (c * cpce) / kGroup;
        float d = 0.f, xsm = 0.f;
        for (int q = 0; q < cpce; ++q) {
          const int col = c * cpce + q;          // element of x in the interleaved layout
          const float xv = xs[4 * ilv<kCpc>(col / 4, nch) + col % 4];
          const uint32_t word = q / (32 / eb) == 0 ? v.x : q / (32 / eb) == 1 ? v.y : q / (32 / eb) == 2 ? v.z : v.w;
          const uint32_t code = (word >> (eb * (q % (32 / eb)))) & ((1u << eb) - 1u);
          d = fmaf((float)code, xv, d);
          xsm += xv;
        }
        a = fmaf(bf16_to_f32(L.sh_eg.scales[gg]), d, fmaf(bf16_to_f32(L.sh_eg.biases[gg]), xsm, a));
      }
      a = wave_sum(a);
      if (lane == 0) st_coh(P.sg + t, a);
    }
    drain();
    __syncthreads();
    if (tid == 0) {
      int* tl = tok_lines(t);
      if (arrive(tl, r, upt))
        __hip_atomic_store(tl + 2 * (1 + kFan) * kLine, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
    // ------------------------------------------------------------ D unit
    const int d = u - P.g_units;
    const int t = d / P.nc;
    const int c = d - t * P.nc;
    const int r0 = c * kDRows;
    const int nrows = min(kDRows, H - r0);
    const int I = L.I, Is = L.Is;
    const int cpr = I / kCpc;                    // chunks per routed down row
    const int cps = L.has_shared ? Is / kCpc : 0;
    const int tot = K * cpr + cps;               // chunks per output row, all slots
    // slot of every chunk position and the row bases, per lane (chunks q = lane + 64 j)
    int eoff[DCH];                          // expert (or shared) row base, in rows
    int kq[DCH];                            // slot of the chunk, -1 if none
    int cq[DCH];                            // chunk within the slot's row
#pragma unroll
    for (int j = 0; j < DCH; ++j) {
      const int q = lane + kWave * j;
      kq[j] = -1;
      cq[j] = 0;
      eoff[j] = 0;
      if (q < tot) {
        const int k = q < K * cpr ? q / cpr : K;
        kq[j] = k;
        cq[j] = k < K ? q - k * cpr : q - K * cpr;
        if (k < K) {
          const int e = idx[(size_t)t * K + k];
          eoff[j] = (e >= 0 && e < L.E ? e : 0) * H;
        }
      }
    }
    // 1) issue every HBM load: the unit's scales and biases for every slot
    //    (per slot kDRows rows x groups bf16, contiguous), then 2 rows x up to
    //    DCH chunks per lane
    const int gr = I / kGroup, gs = L.has_shared ? Is / kGroup : 0;
    const int sb_r = kDRows * gr * 2 / 16;       // 16-byte words per slot and tensor
    const int sb_s = kDRows * gs * 2 / 16;
    const int n_sb = 2 * (K * sb_r + sb_s);      // all slots, scales and biases
    uint4 sbr[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = tid + 256 * j;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (q < n_sb) {
        const int half = q < K * sb_r + sb_s ? 0 : 1;          // 0: scales, 1: biases
        const int qq = q - half * (K * sb_r + sb_s);
        const int k = qq < K * sb_r ? qq / sb_r : K;
        const int w = k < K ? qq - k * sb_r : qq - K * sb_r;
        size_t base;
        const uint16_t* src;
        if (k < K) {
          const int e = idx[(size_t)t * K + k];
          base = ((size_t)(e >= 0 && e < L.E ? e : 0) * H + r0) * gr;
          src = half ? L.down.biases : L.down.scales;
        } else {
          base = (size_t)r0 * gs;
          src = half ? L.sh_down.biases : L.sh_down.scales;
        }
        if (r0 + kDRows <= H || w * 8 < (H - r0) * (k < K ? gr : gs))
          v = reinterpret_cast<const uint4*>(src + base)[w];
      }
      sbr[j] = v;
    }
    uint4 wv[2][DCH];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int rl = wid * 2 + rr;
#pragma unroll
      for (int j = 0; j < DCH; ++j) {
        const bool ok = kq[j] >= 0 && rl < nrows;
        const bool sh = kq[j] == K;
        const uint32_t* base = sh ? L.sh_down.q : L.down.q;
        const int wpr = (sh ? Is : I) / (32 / BITS);
        wv[rr][j] = ok ? reinterpret_cast<const uint4*>(base + (size_t)(eoff[j] + r0 + rl) * wpr)[cq[j]]
                       : make_uint4(0, 0, 0, 0);
      }
    }
    // per-slot weights (routing weights; sigmoid(sg) for the shared slot) and
    // whether the token has an out-of-range expert index (its rows become NaN)
    __shared__ float wk[17];
    __shared__ int bad;
    if (tid == 0) bad = 0;
    __syncthreads();
    if (tid < K) {
      const int e = idx[(size_t)t * K + tid];
      wk[tid] = wts[(size_t)t * K + tid];
      if (e < 0 || e >= L.E) atomicOr(&bad, 1);
    }
    // 2) wait for token t's h, then stage it (coherent loads) with chunk sums
    if (tid == 0) {
      if (!wait_flag(tok_lines(t) + 2 * (1 + kFan) * kLine)) atomicOr(err, 1);
      if (L.has_shared) wk[K] = 1.0f / (1.0f + __expf(-ld_coh(P.sg + t)));
    }
    __syncthreads();
    float* hs = smem;                            // [S][Imax]
    float* hsum = hs + (size_t)P.S * P.Imax;     // [S][Imax/kCpc]
    // bf16 scales then biases: slot k < K at k*kDRows*gr, shared after them
    uint16_t* sbl = reinterpret_cast<uint16_t*>(hsum + (size_t)P.S * P.Imax / 16);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = tid + 256 * j;
      if (q < n_sb) reinterpret_cast<uint4*>(sbl)[q] = sbr[j];
    }
    {
      // all coherent loads of a batch in flight before any is consumed
      const uint64_t* h2 = reinterpret_cast<const uint64_t*>(P.h + (size_t)t * P.S * P.Imax);
      const int n2 = P.S * P.Imax / 2;
      constexpr int kB = 16;
      for (int b0 = 0; b0 < n2; b0 += 256 * kB) {
        uint64_t r[kB];
#pragma unroll
        for (int j = 0; j < kB; ++j) {
          const int i = b0 + tid + 256 * j;
          r[j] = i < n2 ? ld_coh64(h2 + i) : 0ull;
        }
#pragma unroll
        for (int j = 0; j < kB; ++j) {
          const int i = b0 + tid + 256 * j;      // floats 2i, 2i+1 of the token's h
          if (i < n2) {
            const int k = (2 * i) / P.Imax;
            const int e = 2 * i - k * P.Imax;    // element within the slot
            const int nk = (k == K ? Is : I) / kCpc;
            if (e < nk * kCpc) {
              float* dst = hs + (size_t)k * P.Imax + 4 * ilv<kCpc>(e / 4, nk) + e % 4;
              *reinterpret_cast<uint64_t*>(dst) = r[j];
            }
          }
        }
      }
    }
    __syncthreads();
    // chunk sums of every slot, one (slot, chunk) pair per thread
    for (int q = tid; q < tot; q += blockDim.x) {
      const int k = q < K * cpr ? q / cpr : K;
      const int cc = k < K ? q - k * cpr : q - K * cpr;
      const int nk = k < K ? cpr : cps;
      const float4* a4 = reinterpret_cast<const float4*>(hs + (size_t)k * P.Imax);
      float sum = 0.f;
#pragma unroll
      for (int f = 0; f < kCpc / 4; ++f) {
        const float4 v = a4[f * nk + cc];
        sum += (v.x + v.y) + (v.z + v.w);
      }
      hsum[(size_t)k * (P.Imax / kCpc) + cc] = sum;
    }
    __syncthreads();
    // 3) two rows per wave: per-lane partials over the lane's chunks, then
    //    one transposed reduction
    float pv[2];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int rl = wid * 2 + rr;
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < DCH; ++j) {
        const int k = kq[j];
        if (k >= 0 && rl < nrows) {
          const bool sh = k == K;
          const int Ik = sh ? Is : I;
          const int gpr = Ik / kGroup;
          const float4* hk = reinterpret_cast<const float4*>(hs + (size_t)k * P.Imax);
          const float dd = chunk_dot<BITS>(wv[rr][j], hk + cq[j], Ik / kCpc);
          const int gi = (sh ? K * kDRows * gr : k * kDRows * gr) + rl * gpr + (cq[j] * kCpc) / kGroup;
          const int boff = K * kDRows * gr + kDRows * gs;    // biases follow all scales
          const float part = fmaf(bf16_to_f32(sbl[gi]), dd,
                                  bf16_to_f32(sbl[boff + gi]) * hsum[(size_t)k * (P.Imax / kCpc) + cq[j]]);
          acc = fmaf(wk[k], part, acc);
        }
      }
      pv[rr] = acc;
    }
    const float tsum = treduce<2, 32>(pv, lane);
    if ((lane & 31) == 0) {
      const int rl = wid * 2 + tindex<2, 32>(lane);
      if (rl < nrows) {
        float v = bad ? __builtin_nanf("") : tsum;
        if (residual) v += residual[(size_t)t * H + r0 + rl];
        y[(size_t)t * H + r0 + rl] = v;
      }
    }
    // the last D unit of token t to arrive lowers the ready flag (every D unit
    // of the token has finished waiting on it)
    __syncthreads();
    if (tid == 0) {
      int* tl = tok_lines(t);
      if (arrive(tl + (1 + kFan) * kLine, c, P.nc))
        __hip_atomic_store(tl + 2 * (1 + kFan) * kLine, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

DecPlan make_dec_plan(const DecodeLayer& L, int M, int K, void* ws, size_t* bytes) {
  DecPlan P{};
  P.M = M;
  P.K = K;
  P.S = K + (L.has_shared ? 1 : 0);
  P.P = M * P.S;
  P.Imax = L.has_shared && L.Is > L.I ? L.Is : L.I;
  P.ng_routed = (L.I + kGRows - 1) / kGRows;
  P.ng_shared = L.has_shared ? (L.Is + kGRows - 1) / kGRows : 0;
  P.g_units = M * (K * P.ng_routed + P.ng_shared);
  P.nc = (L.H + kDRows - 1) / kDRows;
  P.d_units = M * P.nc;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  size_t off = 0;
  const size_t n_ctr = (size_t)kLine * (1 + (size_t)kCtrLines * M);
  char* base = reinterpret_cast<char*>(ws);
  P.ctr = reinterpret_cast<int*>(base + off);
  off += al(sizeof(int) * n_ctr);
  P.h = reinterpret_cast<float*>(base + off);
  off += al(sizeof(float) * (size_t)P.P * P.Imax);
  P.sg = reinterpret_cast<float*>(base + off);
  off += al(sizeof(float) * (size_t)M);
  if (bytes) *bytes = off;
  return P;
}

size_t decode_ws_bytes(const DecodeLayer& L, int M, int K) {
  size_t b = 0;
  make_dec_plan(L, M, K, nullptr, &b);
  return b;
}

size_t decode_lds_bytes(const DecodeLayer& L, int K) {
  // G: x (H floats) + chunk sums (<= H/16) + 4 x 16 rows x groups bf16;
  // D: h of all S slots (S x Imax floats) + their chunk sums (<= 1/16 of that)
  const size_t g = sizeof(float) * (L.H + L.H / 16) + 2 * 4 * kGRows * (L.H / kGroup);
  const int S = K + (L.has_shared ? 1 : 0);
  const int Im = L.has_shared && L.Is > L.I ? L.Is : L.I;
  const size_t d = sizeof(float) * ((size_t)S * Im + (size_t)S * Im / 16) +
                   2 * 2 * (size_t)kDRows * (K * (L.I / kGroup) + (L.has_shared ? L.Is / kGroup : 0));
  return (g > d ? g : d) + 64;
}

// 16-byte chunks per lane of a D row (all slots), rounded up to 1,2,3,4,6,8
static int d_ch(const DecodeLayer& L, int K) {
  const int cpc = 128 / L.gate.bits;
  const int tot = K * (L.I / cpc) + (L.has_shared ? L.Is / cpc : 0);
  const int n = (tot + kWave - 1) / kWave;
  return n <= 1 ? 1 : n <= 2 ? 2 : n <= 3 ? 3 : n <= 4 ? 4 : n <= 6 ? 6 : n <= 8 ? 8 : 0;
}

// chunks per lane of a G row (1, 2 or 4) for H columns at BITS; 0 if more
static int g_cpl(int H, int bits) {
  const int nch = H / (128 / bits);
  return nch <= kWave ? 1 : nch <= 2 * kWave ? 2 : nch <= 4 * kWave ? 4 : 0;
}

// limits of this kernel: x at most 4096 floats (one 16-byte word per thread
// per 1024), G rows of at most 4 chunks per lane, D rows (all slots) of at
// most 8 chunks per lane, the shared expert at the routed experts' bit width,
// a G unit's scales/biases within one 16-byte word per thread, and the LDS
bool decode_supported(const DecodeLayer& L, int K) {
  const int b = L.gate.bits;
  if (L.H > 4096 || !g_cpl(L.H, b)) return false;
  if (kGRows * (L.H / kGroup) * 2 / 16 > 256) return false;
  if (L.has_shared) {
    if (L.sh_gate.bits != b) return false;
    if (L.sh_eg.bits != 2 && L.sh_eg.bits != 4 && L.sh_eg.bits != 8) return false;
  }
  if (!d_ch(L, K)) return false;
  // the D unit stages its scales/biases with at most two 16-byte words per thread
  const int words = 2 * kDRows * (K * (L.I / kGroup) + (L.has_shared ? L.Is / kGroup : 0)) * 2 / 16;
  if (words > 2 * 256) return false;
  return decode_lds_bytes(L, K) <= 160 * 1024;
}

template <int B, int CPL, int DCH>
static void run_fused(const DecodeLayer& L, const DecPlan& P, const float* x, const int32_t* idx,
                      const float* w, const float* residual, float* y, hipStream_t s) {
  const size_t lds = decode_lds_bytes(L, P.K);
  hipLaunchKernelGGL((k_dec_fused<B, CPL, DCH>), dim3(P.g_units + P.d_units), dim3(256), lds, s,
                     L, P, x, idx, w, residual, y);
}

int launch_decode_forward(const DecodeLayer& L, const float* x, const int32_t* idx, const float* w,
                          int M, int K, const float* residual, float* y, void* ws, hipStream_t s) {
  const DecPlan P = make_dec_plan(L, M, K, ws, nullptr);
  const int b = L.gate.bits;
  const int cpl = g_cpl(L.H, b);
  const int dch = d_ch(L, K);
#define MOEQ_DEC(B_, C_, D_)                                    \
  if (b == B_ && cpl == C_ && dch == D_) {                     \
    run_fused<B_, C_, D_>(L, P, x, idx, w, residual, y, s);    \
    return 0;                                                  \
  }
#define MOEQ_DEC_PW(B_, C_) MOEQ_DEC(B_, C_, 1) MOEQ_DEC(B_, C_, 2) MOEQ_DEC(B_, C_, 3) \
  MOEQ_DEC(B_, C_, 4) MOEQ_DEC(B_, C_, 6) MOEQ_DEC(B_, C_, 8)
#define MOEQ_DEC_C(B_) MOEQ_DEC_PW(B_, 1) MOEQ_DEC_PW(B_, 2) MOEQ_DEC_PW(B_, 4)
  MOEQ_DEC_C(8)
  MOEQ_DEC_C(4)
  MOEQ_DEC_C(2)
#undef MOEQ_DEC_C
#undef MOEQ_DEC_PW
#undef MOEQ_DEC
  return -9;
}

}  // namespace moeq
