// Decode step (fp32 activations, small M) as ONE launch: router, top-K and
// the selected experts, or the experts alone for given indices.
//
// The step (markbaseengine MOE_ROUTER_WORKS_BREAKTHROUGH, "Forward Pass
// Sequence": router projection, softmax, top-K, expertFusedGateUp,
// expertDown, accumulateResults; flash-moe-inference kernels swiglu and
// moe_combine_residual):
//   h_k = silu(Gate_e x) * (Up_e x),   y = sum_k w_k Down_e h_k
//         (+ sigmoid(sg . x) * FFN_shared(x)) (+ residual).
//
// Work units by block index, every unit 8 waves:
//   R units  (routing in the launch only; 8 router rows each): fp64 logits of
//            all M tokens, published one by one; the last R unit collects
//            them, selects the top-K of every token and publishes each
//            (expert + 1, weight) pair as one 64-bit word (0 means "not yet").
//   G units  (pair p = token*S + slot, 16 intermediate rows): gate and up rows
//            of the pair's expert against x, SwiGLU, h[p][i]; the first G unit
//            of a shared-expert pair also computes the shared_expert_gate
//            logit.  With routing in the launch a G unit stages x and its chunk
//            sums while it waits for its expert index.  Each G unit counts its
//            arrival for token t; the one that completes the count raises
//            ready[t].
//   D units  (token t, 8 output rows): issue the weight loads of their rows
//            for all S slots (the shared expert's before the routed experts'
//            indices are known), wait for ready[t], stage h of all S pairs in
//            LDS and produce whole output rows,
//            y = sum_k w_k Down_k h_k (+ sigmoid(sg) Down_sh h_sh) (+ residual),
//            with one fixed reduction order, so results are bitwise
//            reproducible and no data crosses blocks twice.  The last D unit of
//            a token to arrive lowers ready[t] and clears the token's published
//            indices for the next launch.
// Workgroups are dispatched in index order within each XCD, so when a unit
// runs, every unit of a lower index on its XCD has been dispatched; a unit
// only ever waits for units of lower index, so each wait ends.  Waits are
// bounded anyway: one that exceeds its spin limit records an error word in the
// workspace and gives up instead of hanging.  Arrivals are counted with
// two-level counters (see arrive()).
//
// Latency is what bounds a decode layer, so every unit issues all of its HBM
// loads (weight rows, and the rows' bf16 scales and biases, staged through
// LDS) as soon as their addresses are known and before it touches any result,
// and units are sized so that a whole layer's blocks are resident at once.
// Rows are streamed in 16-byte chunks (128/BITS codes, never straddling a
// 64-column group); a chunk contributes s*(sum_j q_j a_j) + b*(sum_j a_j)
// with the activation's chunk sums precomputed once per block in LDS.
#include "common.h"
#include "launch.h"
#include "topk.h"
#include "decode_common.h"

namespace moeq {

constexpr int kThreads = 512;              // every unit is 8 waves
constexpr int kWaves = kThreads / kWave;
constexpr int kGRows = 16;                 // intermediate rows per G unit (two per wave)
constexpr int kDRows = kWaves;             // output rows per D unit (one per wave)
constexpr int kRRows = kWaves / 2;         // router rows per R unit (two waves per row)
constexpr int kSpinLimit = 1 << 26;
constexpr int kLine = kLineInts;
constexpr int kRep = 64;      // copies of every flag that many units poll
// per token: G arrival counter lines, D arrival counter lines
constexpr int kCtrLines = 2 * (1 + kFan);
constexpr int kHCopies = 8;   // copies of h (one per XCD; the down units read their XCD's): spreads the
                              // reads of all D units of a token over more memory channels

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


__device__ __forceinline__ int ld_coh_i(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh_i(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Polling.  Every poll is a coherent load that the memory side serves; many
// units polling one line at a high rate would take a share of that line's
// memory channel away from the weight stream.  So every flag that many units
// wait on exists in kRep copies, one copy per block of flags, the blocks 4 KB
// + 256 B apart so that the copies fall on different channels (a unit polls
// copy unit % kRep), and polls are spaced by s_sleep.

__device__ __forceinline__ uint64_t ld_coh_u64(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// lanes < n of one wave wait until p[lane] != 0; returns the lane's value
// (0, and an error bit, if the spin limit hit)
__device__ __forceinline__ uint64_t wave_wait_nonzero(const uint64_t* p, int n, int lane, int* err) {
  uint64_t v = 0;
  for (int i = 0; i < kSpinLimit; ++i) {
    if (lane < n) v = ld_coh_u64(p + lane);
    if (__all(lane >= n || v != 0)) return v;
    __builtin_amdgcn_s_sleep(2);
  }
  if (lane == 0) atomicOr(err, 2);
  return v;
}

// wait (one thread) until *flag != 0; returns false if the spin limit hit
__device__ __forceinline__ bool wait_flag(int* flag) {
  for (int i = 0; i < kSpinLimit; ++i) {
    if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return true;
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}

// the token's route line in copy `rep`: word k = (expert + 1) << 32 | the
// routing weight's fp32 bits, 0 while not routed (one 64-bit store publishes
// both halves together)
__device__ __forceinline__ uint64_t* route_line(const DecPlan& P, int rep, int t) {
  return reinterpret_cast<uint64_t*>(P.idx_c + (size_t)rep * P.rstride + (size_t)t * kLine);
}
__device__ __forceinline__ int* ready_line(const DecPlan& P, int rep, int t) {
  return P.ready + (size_t)rep * P.rstride + (size_t)t * kLine;
}

// ---- fp64 wave sum on VALU exchanges (DPP and gfx950 permlane swaps) -------
template <int M>
__device__ __forceinline__ double xchg_d(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  if constexpr (M >= 16) {
    const auto rl = M == 32 ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                            : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto rh = M == 32 ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                            : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    // r[0], r[1]: this lane's and its partner's value, in lane order
    const double a = __longlong_as_double((long long)(((uint64_t)rh[0] << 32) | rl[0]));
    const double b = __longlong_as_double((long long)(((uint64_t)rh[1] << 32) | rl[1]));
    return a + b;
  } else {
    constexpr int ctrl = M == 1 ? 0xB1 : M == 2 ? 0x4E : M == 4 ? 0x141 : 0x140;
    lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)lo, ctrl, 0xF, 0xF, false);
    hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)hi, ctrl, 0xF, 0xF, false);
    return v + __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
  }
}
// every lane gets the sum of the wave's 64 values (mirror steps: see treduce)
__device__ __forceinline__ double wave_sum_d(double v) {
  v = xchg_d<32>(v);
  v = xchg_d<16>(v);
  v = xchg_d<8>(v);
  v = xchg_d<4>(v);
  v = xchg_d<2>(v);
  return xchg_d<1>(v);
}



// ------------------------------------------------------------------ R unit
// top-K of at most 64*PER keys by one wave, keys held in registers: K rounds
// of a wave maximum, the owner of each winner dropping it (keys are unique)
template <int PER>
__device__ __forceinline__ void wave_topk(const uint64_t* keys, int E, int K, int lane, int* sel) {
  uint64_t kk[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + kWave * i;
    kk[i] = e < E ? keys[e] : 0ull;      // 0 is below every key
  }
  for (int r = 0; r < K; ++r) {
    uint64_t mx = kk[0];
#pragma unroll
    for (int i = 1; i < PER; ++i) mx = kk[i] > mx ? kk[i] : mx;
    mx = wave_max_u64(mx);
#pragma unroll
    for (int i = 0; i < PER; ++i) kk[i] = kk[i] == mx ? 0ull : kk[i];
    if (lane == 0) sel[r] = 1023 - (int)(mx & 0x3FFull);
  }
}

// top-K of token m from keys/vals in LDS (E <= 1024), all threads of the
// block: selection by rank as in topk.h, candidates ranked by four threads
// each; publishes the weights into every route-line copy, drains, then the
// indices, and writes the caller's outputs.
// WIDE: allow the one-wave selection up to 512 experts (16 more registers)
template <bool WIDE>
__device__ __forceinline__ void route_select(const uint64_t* keys, const double* vals, int E,
                                             int K, int renorm, const DecPlan& P, const RouteIn& R,
                                             int m, int par) {
  __shared__ uint64_t cand[kWaves * kMaxTopK];
  __shared__ int sel[kMaxTopK];
  __shared__ double ex[kMaxTopK];
  __shared__ double red[kWaves];
  __shared__ double s_tot;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  if (E <= kThreads / 4) {               // up to 128 experts: rank every key, one quad per key
    const int a = tid >> 2, part = tid & 3;
    const uint64_t ka = a < E ? keys[a] : 0ull;
    int rank = 0;
#pragma unroll 8
    for (int j = part; j < E; j += 4) rank += keys[j] > ka;
    rank += __builtin_amdgcn_mov_dpp(rank, 0xB1, 0xF, 0xF, false);
    rank += __builtin_amdgcn_mov_dpp(rank, 0x4E, 0xF, 0xF, false);
    if (part == 0 && a < E && rank < K) sel[rank] = a;
  } else if (WIDE && E <= 8 * kWave) {   // up to 512
    if (wid == 0) wave_topk<8>(keys, E, K, lane, sel);
  } else {
  const int nc = kWaves * K;             // candidate slots, K per wave
  if (tid < nc) cand[tid] = 0ull;        // 0 is below every key
  __syncthreads();
  // 1) per wave: the keys of its part whose rank inside the part is < K, at
  //    their rank (keys are unique, so the positions are too)
  const int q = (E + kWaves - 1) / kWaves;
  const int lo = min(E, wid * q), hi = min(E, lo + q);
  for (int a = lo + lane; a < hi; a += kWave) {
    const uint64_t ka = keys[a];
    int rank = 0;
#pragma unroll 4
    for (int j = lo; j < hi; ++j) rank += keys[j] > ka;
    if (rank < K) cand[wid * K + rank] = ka;
  }
  __syncthreads();
  // 2) rank of every candidate among the candidates: four threads (one quad)
  //    per candidate, each over a quarter, summed across the quad
  {
    const int c = tid >> 2, part = tid & 3;
    const uint64_t kc = c < nc ? cand[c] : 0ull;
    int rank = 0;
#pragma unroll 4
    for (int j = part; j < nc; j += 4) rank += cand[j] > kc;
    rank += __builtin_amdgcn_mov_dpp(rank, 0xB1, 0xF, 0xF, false);
    rank += __builtin_amdgcn_mov_dpp(rank, 0x4E, 0xF, 0xF, false);
    if (part == 0 && c < nc && kc != 0ull && rank < K) sel[rank] = 1023 - (int)(kc & 0x3FFull);
  }
  }
  __syncthreads();
  // 3) weights in fp64: p[idx] / sum p[idx] (renorm, summed in slot order) or
  //    p[idx] / sum over all E (fixed order), with p relative to the maximum
  const double mx = vals[sel[0]];
  if (tid < K) ex[tid] = exp(vals[sel[tid]] - mx);
  if (!renorm) {
    double part = 0.0;
    for (int e = tid; e < E; e += kThreads) part += exp(vals[e] - mx);
    part = wave_sum_d(part);
    if (lane == 0) red[wid] = part;
  }
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
    if (renorm)
      for (int k = 0; k < K; ++k) tot += ex[k];
    else
      for (int w = 0; w < kWaves; ++w) tot += red[w];
    s_tot = tot;
  }
  __syncthreads();
  for (int i = tid; i < kRep * K; i += kThreads) {
    const int rep = i / K, k = i - rep * K;
    const float w = (float)(ex[k] / s_tot);
    if (rep == 0) {
      R.idx_out[(size_t)m * K + k] = sel[k];
      R.w_out[(size_t)m * K + k] = w;
    }
    const uint32_t hi = ((uint32_t)par << 31) | (uint32_t)(sel[k] + 1);
    st_coh_u64(route_line(P, rep, m) + k, ((uint64_t)hi << 32) | __float_as_uint(w));
  }
}

// Router rows (8-bit) against x for all M tokens in fp64: the fp32
// dequantized weight widened exactly, fp64 products and sums, as the oracle
// defines the logits.  The R unit completing the arrivals selects.
// NORM: the rows see h = r * (x . g) with r = 1/sqrt(mean(x^2) + eps) per token
// (RMSNorm): x . g is staged, each token's mean square reduced over the block,
// and r applied to the finished logit.
template <bool WIDE, bool NORM>
__device__ __forceinline__ void route_unit(const DecodeLayer L, const DecPlan P, const RouteIn R,
                                           const float* __restrict__ x, int u) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int E = L.E, H = L.H, M = P.M, K = P.K;
  // two waves per row: wave half h takes the row's chunks lane + 64 (2j + h)
  const int e = u * kRRows + wid / 2, h = wid & 1;
  const int nch = H / 16;                 // 16 codes per chunk at 8 bits
  const int rsh = __builtin_ctz((unsigned)R.W.group_size);   // log2 of the group size
  const int gpr = H >> rsh;
  const bool row_ok = e < E;
  __shared__ double part[kFusedMaxM][kRRows];
  // Loads use clamped, always valid addresses and no branches, so they all
  // issue back to back; lanes past the row's end are never used.
  const int er = min(e, E - 1);
  // the selector's epoch word (its parity picks the launch's h buffer), read
  // now so the load overlaps the router rows
  const int epoch = u == P.r_units - 1 ? ld_coh_i(P.epoch) : 0;
  uint4 rv[2];
  uint32_t rsb[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = min(lane + kWave * (2 * j + h), nch - 1);
    rv[j] = reinterpret_cast<const uint4*>(R.W.q + (size_t)er * (H / 4))[c];
    rsb[j] = (uint32_t)R.W.scales[(size_t)er * gpr + ((c * 16) >> rsh)] |
             ((uint32_t)R.W.biases[(size_t)er * gpr + ((c * 16) >> rsh)] << 16);
  }
  // x of every token in LDS, chunk-interleaved (float4 f of chunk c at f*nch+c)
  float4* xl = reinterpret_cast<float4*>(smem);
  __shared__ float s_ss[NORM ? kWaves : 1][kFusedMaxM];
  float ss[kFusedMaxM];
#pragma unroll
  for (int m = 0; m < kFusedMaxM; ++m) ss[m] = 0.f;
  for (int i = tid; i < M * (H / 4); i += kThreads) {
    const int m = i / (H / 4), ii = i - m * (H / 4);
    float4 v = reinterpret_cast<const float4*>(x)[i];
    if constexpr (NORM) {
      const float4 g = reinterpret_cast<const float4*>(P.norm_w)[ii];
      const float q = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
#pragma unroll
      for (int mm = 0; mm < kFusedMaxM; ++mm) ss[mm] += mm == m ? q : 0.f;
      v = make_float4(v.x * g.x, v.y * g.y, v.z * g.z, v.w * g.w);
    }
    xl[m * (H / 4) + (ii % 4) * nch + ii / 4] = v;
  }
  if constexpr (NORM) {
#pragma unroll
    for (int m = 0; m < kFusedMaxM; ++m) {
      if (m < M) {
        const float v = wave_sum(ss[m]);
        if (lane == 0) s_ss[wid][m] = v;
      }
    }
  }
  float rs[2], rb[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    rs[j] = bf16_to_f32(rsb[j] & 0xFFFFu);
    rb[j] = bf16_to_f32(rsb[j] >> 16);
  }
  __syncthreads();
  // per lane and token, its chunks as independent fp64 chains, elements in
  // order; a weight is dequantized once for all tokens; one chunk at a time
  // (the scheduling barrier keeps the compiler from hoisting every chunk's
  // fp64 operands at once)
  double acc[kFusedMaxM][2];
#pragma unroll
  for (int m = 0; m < kFusedMaxM; ++m)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[m][j] = 0.0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = lane + kWave * (2 * j + h);
    if (row_ok && c < nch) {
      const uint32_t wd[4] = {rv[j].x, rv[j].y, rv[j].z, rv[j].w};
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        double w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = (double)fmaf(rs[j], (float)((wd[f] >> (8 * q)) & 0xFFu), rb[j]);
#pragma unroll
        for (int m = 0; m < kFusedMaxM; ++m) {
          if (m < M) {
            const float4 xv = xl[m * (H / 4) + f * nch + c];
            acc[m][j] = fma(w[0], (double)xv.x, acc[m][j]);
            acc[m][j] = fma(w[1], (double)xv.y, acc[m][j]);
            acc[m][j] = fma(w[2], (double)xv.z, acc[m][j]);
            acc[m][j] = fma(w[3], (double)xv.w, acc[m][j]);
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // the two halves of a row meet in LDS; the even wave publishes the logit
  double wsum[kFusedMaxM];
#pragma unroll
  for (int m = 0; m < kFusedMaxM; ++m) {
    wsum[m] = 0.0;
    if (m < M) {
      wsum[m] = wave_sum_d(acc[m][0] + acc[m][1]);
      if (h == 1 && lane == 0) part[m][wid / 2] = wsum[m];
    }
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < kFusedMaxM; ++m) {
    if (m < M && h == 0 && lane == 0 && row_ok) {
      double tot = wsum[m] + part[m][wid / 2];
      if constexpr (NORM) {
        float sq = 0.f;
        for (int w = 0; w < kWaves; ++w) sq += s_ss[w][m];
        tot *= 1.0 / sqrt((double)sq / H + (double)P.norm_eps);
      }
      // published as the complement of its bits: zero means "not written yet"
      // (the complement of a finite double is never zero)
      st_coh_u64(P.logits + (size_t)m * E + e, ~(uint64_t)__double_as_longlong(tot));
    }
  }
  // the last R unit selects: it polls every logit (no counter round trips),
  // clears them for the next launch, and runs the top-K of each token
  if (u != P.r_units - 1) return;
  uint64_t* keys = reinterpret_cast<uint64_t*>(smem);
  double* vals = reinterpret_cast<double*>(keys + E);
  // (the selector is the only reader and writer of the epoch word)
  __syncthreads();                       // x in LDS is no longer read
  for (int m = 0; m < M; ++m) {
    for (int ee = tid; ee < E; ee += kThreads) {
      uint64_t* src = P.logits + (size_t)m * E + ee;
      uint64_t v = 0;
      for (int i = 0; i < kSpinLimit && v == 0; ++i) {
        v = ld_coh_u64(src);
        if (v == 0) __builtin_amdgcn_s_sleep(1);
      }
      if (v == 0) atomicOr(P.ctr, 4);
      st_coh_u64(src, 0);
      const double lg = __longlong_as_double((long long)~v);
      vals[ee] = lg;
      keys[ee] = route_key(lg, ee);
    }
    __syncthreads();
    route_select<WIDE>(keys, vals, E, K, R.renorm, P, R, m, epoch & 1);
    __syncthreads();
  }
  if (tid == 0) {
    st_coh_i(P.epoch, epoch + 1);
    // how much of this launch's h buffer it fills (the launch after next
    // clears that much of it)
    st_coh_i(P.hext + (epoch & 1), (int)((size_t)kHCopies * P.P * P.Imax / 4));
  }
}

// ------------------------------------------------------------------ G unit
// LDS: [x, chunk-interleaved][its chunk sums (<= H/16 floats)][bf16 scales and
// biases of the unit's gate and up rows]
template <int BITS, int CPL, bool FUSED, bool NORM>
__device__ __forceinline__ void gate_up_unit(const DecodeLayer L, const DecPlan P,
                                             const float* __restrict__ x,
                                             const int32_t* __restrict__ idx, int u) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ int s_e, s_par, s_done;
  constexpr int kCpc = 128 / BITS;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int S = P.S, K = P.K, H = L.H;
  const int upt = K * P.ng_routed + (L.has_shared ? P.ng_shared : 0);
  const int t = u / upt;
  const int r = u - t * upt;
  const bool shared = r >= K * P.ng_routed;
  const int k = shared ? K : r / P.ng_routed;
  const int g = shared ? r - K * P.ng_routed : r - k * P.ng_routed;
  const int p = t * S + k;
  const int I = shared ? L.Is : L.I;
  const QT Gq = shared ? L.sh_gate : L.gate;
  const QT Uq = shared ? L.sh_up : L.up;
  const int i_base = g * kGRows;                    // the unit's first row
  const int nrows = min(kGRows, I - i_base);
  const int nch = H / kCpc;                         // chunks per row
  const int wpr = H / (32 / BITS);                  // words per row
  const int esh = __builtin_ctz((unsigned)L.gate.group_size);  // log2 group size, every expert matrix
  const int gpr = H >> esh;                         // groups per row
  const int x16 = H / 4;
  const int sb16 = kGRows * gpr * 2 / 16;           // 16-byte words per scale/bias tensor
  float* xs = smem;
  float* xsum = xs + H;
  // (the sums' region is padded to 16 bytes: the scale words are stored as uint4)
  uint16_t* sbl = reinterpret_cast<uint16_t*>(xsum + pad4(H / 16));   // [4][kGRows * gpr]
  float4* x4 = reinterpret_cast<float4*>(xs);

  uint4 xr[2], gr[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = tid + j * kThreads;
    xr[j] = reinterpret_cast<const uint4*>(x + (size_t)t * H)[min(i, x16 - 1)];
    if constexpr (NORM) gr[j] = reinterpret_cast<const uint4*>(P.norm_w)[min(i, x16 - 1)];
  }
  // NORM: x . g is staged and the token's r = 1/sqrt(mean(x^2) + eps) scales
  // the finished gate and up sums (both are linear in the row)
  __shared__ float s_gss[NORM ? kWaves : 1];
  // the first shared-expert unit of a token also computes the token's
  // shared_expert_gate logit (one row of H, its own bits): one 16-byte chunk
  // per thread (H * bits / 128 <= kThreads), loaded now with the x loads
  const bool sgu = shared && g == 0;                // uniform over the block
  const int eb = L.sh_eg.bits, cpce = 128 / eb, nche = H / cpce;
  uint4 egv = make_uint4(0u, 0u, 0u, 0u);
  uint32_t egsb = 0u;
  if (sgu) {
    const int c = min(tid, nche - 1);
    const int gg = group_of(c * cpce, L.sh_eg.group_size);
    egv = reinterpret_cast<const uint4*>(L.sh_eg.q)[c];
    egsb = (uint32_t)L.sh_eg.scales[gg] | ((uint32_t)L.sh_eg.biases[gg] << 16);
  }
  bool valid = true;
  size_t erow = 0;                                  // first row of the expert
  if constexpr (FUSED) {
    // x and its chunk sums while the router runs, then the expert index
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = tid + j * kThreads;
      if (i < x16) {
        float4 v = reinterpret_cast<const float4&>(xr[j]);
        if constexpr (NORM) {
          const float4 g = reinterpret_cast<const float4&>(gr[j]);
          ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
          v = make_float4(v.x * g.x, v.y * g.y, v.z * g.z, v.w * g.w);
        }
        x4[ilv<kCpc>(i, nch)] = v;
      }
    }
    if constexpr (NORM) {
      ss = wave_sum(ss);
      if (lane == 0) s_gss[wid] = ss;
    }
    __syncthreads();
    chunk_sums<kCpc>(x4, xsum, nch);
    if (wid == 0 && !shared) {
      const uint64_t v = wave_wait_nonzero(route_line(P, u % kRep, t) + k, 1, lane, P.ctr);
      if (lane == 0) {
        s_e = (int)((v >> 32) & 0x7FFFFFFFu) - 1;
        s_par = (int)(v >> 63);
      }
    }
    __syncthreads();
    if (!shared) erow = (size_t)min(max(s_e, 0), L.E - 1) * L.I;
  } else {
    if (!shared) {
      const int e = idx[(size_t)t * K + k];
      valid = e >= 0 && e < L.E;
      erow = (size_t)(valid ? e : 0) * L.I;
    }
  }
  // every HBM load of the unit, scales/biases first (rows x groups bf16,
  // contiguous per tensor), then 2 rows x (gate, up) per wave; clamped,
  // always valid addresses and no branches, so they all issue back to back
  uint4 sbr;
  {
    const size_t o = (erow + i_base) * gpr;
    const int qq = min(tid, 4 * sb16 - 1);
    const int q = qq / sb16, w = qq - q * sb16;
    const uint16_t* src = q == 0 ? Gq.scales : q == 1 ? Gq.biases : q == 2 ? Uq.scales : Uq.biases;
    sbr = reinterpret_cast<const uint4*>(src + o)[w];
  }
  uint4 wg[2][CPL], wu[2][CPL];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int i = wid * 2 + rr;
    const size_t row = erow + i_base + min(i, nrows - 1);
    const uint4* g4 = reinterpret_cast<const uint4*>(Gq.q + row * wpr);
    const uint4* u4 = reinterpret_cast<const uint4*>(Uq.q + row * wpr);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = min(lane + kWave * j, nch - 1);
      wg[rr][j] = g4[c];
      wu[rr][j] = u4[c];
    }
  }
  // done with the route words: count this reader (the last one clears
  // them); the counter round trips overlap the loads just issued
  bool last_reader = false;
  if (FUSED && !shared && tid == 0)
    last_reader = arrive(P.ctr + (size_t)kLine * (1 + (size_t)t * kCtrLines) + (1 + kFan) * kLine, r,
                         upt + P.nc);
  if constexpr (!FUSED) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = tid + j * kThreads;
      if (i < x16) x4[ilv<kCpc>(i, nch)] = reinterpret_cast<const float4&>(xr[j]);
    }
  }
  if (tid < 4 * sb16) reinterpret_cast<uint4*>(sbl)[tid] = sbr;
  __syncthreads();
  if constexpr (!FUSED) {
    chunk_sums<kCpc>(x4, xsum, nch);
    __syncthreads();
  }
  // the wave's two rows: per-lane partials, then one transposed reduction
  float pg[2], pu[2];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int i = wid * 2 + rr;
    float ag = 0.f, au = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + kWave * j;
      if (c < nch) {
        const int grp = i * gpr + ((c * kCpc) >> esh);
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
  const float gsum = treduce<2, 32>(pg, lane);
  const float usum = treduce<2, 32>(pu, lane);
  if constexpr (FUSED) {
    if (shared) {
      // the shared expert does not wait for routing; it learns the launch's
      // parity from the route words now, and counts itself as their reader
      if (wid == 0) {
        const uint64_t v = wave_wait_nonzero(route_line(P, u % kRep, t), 1, lane, P.ctr);
        if (lane == 0) {
          s_par = (int)(v >> 63);
          s_done = arrive(P.ctr + (size_t)kLine * (1 + (size_t)t * kCtrLines) + (1 + kFan) * kLine, r,
                          upt + P.nc);
        }
      }
      __syncthreads();
    }
  }
  float rn = 1.f;
  if constexpr (NORM) {
    float sq = 0.f;
    for (int w = 0; w < kWaves; ++w) sq += s_gss[w];
    rn = (float)(1.0 / sqrt((double)sq / H + (double)P.norm_eps));
  }
  if ((lane & 31) < kHCopies) {         // every lane of a half holds its row's sum
    const int i = wid * 2 + tindex<2, 32>(lane);
    const float hv = valid ? silu(rn * gsum) * (rn * usum) : __builtin_nanf("");
    if (i < nrows) {
      const size_t at = (size_t)(lane & 31) * P.P * P.Imax + (size_t)p * P.Imax + i_base + i;
      if constexpr (FUSED)   // complemented bits: 0 means "not written in this launch"
        st_coh_i(reinterpret_cast<int*>(P.hb) + (size_t)s_par * P.hreg + at,
                 (int)~__float_as_uint(hv));
      else
        st_coh(P.h + at, hv);
    }
  }
  if (sgu) {
    // the shared_expert_gate logit: this thread's chunk, then the block's sum
    // in wave order
    __shared__ float sgp[kWaves];
    float a = 0.f;
    if (tid < nche) {
      float d = 0.f, xsm = 0.f;
      for (int q = 0; q < cpce; ++q) {
        const int col = tid * cpce + q;        // element of x in the interleaved layout
        const float xv = xs[4 * ilv<kCpc>(col / 4, nch) + col % 4];
        const uint32_t word = q / (32 / eb) == 0 ? egv.x : q / (32 / eb) == 1 ? egv.y : q / (32 / eb) == 2 ? egv.z : egv.w;
        const uint32_t code = (word >> (eb * (q % (32 / eb)))) & ((1u << eb) - 1u);
        d = fmaf((float)code, xv, d);
        xsm += xv;
      }
      a = fmaf(bf16_to_f32(egsb & 0xFFFFu), d, bf16_to_f32(egsb >> 16) * xsm);
    }
    a = wave_sum(a);
    if (lane == 0) sgp[wid] = a;
    __syncthreads();
    if (tid == 0) {
      float tot = 0.f;
      for (int w = 0; w < kWaves; ++w) tot += sgp[w];
      tot *= rn;
      if constexpr (FUSED)
        st_coh_i(reinterpret_cast<int*>(P.sgb) + s_par * kFusedMaxM + t, (int)~__float_as_uint(tot));
      else
        st_coh(P.sg + t, tot);
    }
  }
  if constexpr (FUSED) {
    // h goes out with its own "written" marks, so there is nothing to
    // announce; the last reader of the route words clears them
    if (!shared && tid == 0) s_done = last_reader;
    __syncthreads();
    if (s_done)
      for (int i = tid; i < kRep * K; i += kThreads) st_coh_u64(route_line(P, i / K, t) + i % K, 0);
  } else {
    drain();
    __syncthreads();
    if (tid == 0) s_done = arrive(P.ctr + (size_t)kLine * (1 + (size_t)t * kCtrLines), r, upt);
    __syncthreads();
    if (s_done && tid < kRep) st_coh_i(ready_line(P, tid, t), 1);
  }
}

// ------------------------------------------------------------------ D unit
// LDS: [h of all S slots, chunk-interleaved per slot][their chunk sums][bf16
// scales then biases of the unit's rows, slot by slot]
template <int BITS, int DCH, bool FUSED>
__device__ __forceinline__ void down_unit(const DecodeLayer L, const DecPlan P,
                                          const int32_t* __restrict__ idx,
                                          const float* __restrict__ wts,
                                          const float* __restrict__ residual,
                                          float* __restrict__ y, int d) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ float wk[kMaxTopK + 1];
  __shared__ int s_ex[kMaxTopK];
  __shared__ int bad, s_par, s_done, s_zx;
  constexpr int kCpc = 128 / BITS;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int K = P.K, H = L.H;
  const int t = d / P.nc;
  const int c = d - t * P.nc;
  const int r0 = c * kDRows;
  const int nrows = min(kDRows, H - r0);
  const int rl = wid;                          // the wave's row
  const int I = L.I, Is = L.Is;
  const int cpr = I / kCpc;                    // chunks per routed down row
  const int cps = L.has_shared ? Is / kCpc : 0;
  const int tot = K * cpr + cps;               // chunks per output row, all slots
  int* tl = P.ctr + (size_t)kLine * (1 + (size_t)t * kCtrLines);
  // slot and chunk of every chunk position of the lane (q = lane + 64 j)
  // (packed in one register: (slot + 1) << 16 | chunk; slot -1 = no chunk)
  int kc[DCH];
#pragma unroll
  for (int j = 0; j < DCH; ++j) {
    const int q = lane + kWave * j;
    kc[j] = 0;
    if (q < tot) {
      const int k = q < K * cpr ? q / cpr : K;
      kc[j] = ((k + 1) << 16) | (k < K ? q - k * cpr : q - K * cpr);
    }
  }

  if (tid == 0) bad = 0;
  if constexpr (!FUSED) {
    __syncthreads();
    if (tid < K) {
      const int e = idx[(size_t)t * K + tid];
      const bool ok = e >= 0 && e < L.E;
      s_ex[tid] = ok ? e : 0;
      wk[tid] = wts[(size_t)t * K + tid];
      if (!ok) atomicOr(&bad, 1);
    }
  }
  if constexpr (FUSED) {
    if (wid == 0) {
      const uint64_t v = wave_wait_nonzero(route_line(P, d % kRep, t), K, lane, P.ctr);
      if (lane < K) {
        s_ex[lane] = min(max((int)((v >> 32) & 0x7FFFFFFFu) - 1, 0), L.E - 1);
        wk[lane] = __uint_as_float((uint32_t)v);
      }
      if (lane == 0) s_par = (int)(v >> 63);
    }
  }
  __syncthreads();
  // scales and biases of every slot (per slot kDRows rows x groups bf16,
  // contiguous), then the routed chunks
  const int esh = __builtin_ctz((unsigned)L.gate.group_size);  // log2 group size, every expert matrix
  const int gr = I >> esh, gs = L.has_shared ? Is >> esh : 0;
  const int sb_r = kDRows * gr * 2 / 16;       // 16-byte words per slot and tensor
  const int sb_s = kDRows * gs * 2 / 16;
  const int n_sb = 2 * (K * sb_r + sb_s);      // all slots, scales and biases
  // (clamped, always valid addresses and no branches: the loads issue back
  // to back; H is a multiple of kDRows, so every unit has full rows)
  uint4 sbr;
  {
    const int tq = min(tid, n_sb - 1);
    const int half = tq < K * sb_r + sb_s ? 0 : 1;           // 0: scales, 1: biases
    const int qq = tq - half * (K * sb_r + sb_s);
    const int k = qq < K * sb_r ? qq / sb_r : K;
    const int w = k < K ? qq - k * sb_r : qq - K * sb_r;
    const uint16_t* src = k < K ? (half ? L.down.biases : L.down.scales)
                                : (half ? L.sh_down.biases : L.sh_down.scales);
    const size_t base = k < K ? ((size_t)s_ex[k] * H + r0) * gr : (size_t)r0 * gs;
    sbr = reinterpret_cast<const uint4*>(src + base)[w];
  }
  // the residual of the wave's row goes out with the unit's other loads, so
  // the final sum does not wait for it (a wave-uniform address: a scalar
  // load, held in a scalar register)
  float resv = 0.f;
  if (residual)
    resv = residual[(size_t)t * H + r0 + __builtin_amdgcn_readfirstlane(min(rl, nrows - 1))];
  uint4 wv[DCH];
  const int rlc = min(rl, nrows - 1);
#pragma unroll
  for (int j = 0; j < DCH; ++j) {
    const int kj = (kc[j] >> 16) - 1, cj = kc[j] & 0xFFFF;
    const bool sh = kj == K;
    const uint32_t* base = sh ? L.sh_down.q
                              : L.down.q + ((size_t)s_ex[max(kj, 0)] * H) * (I / (32 / BITS));
    const int wpr = (sh ? Is : I) / (32 / BITS);
    wv[j] = reinterpret_cast<const uint4*>(base + (size_t)(r0 + rlc) * wpr)[cj];
  }
  // the extent of the other h buffer's last use (cleared at the end)
  const int zx = FUSED ? ld_coh_i(P.hext + (s_par ^ 1)) : 0;
  // done with the route words: count this reader (the last one clears them);
  // the last wave does it, after its loads are in flight
  bool last_reader = false;
  if (FUSED && tid == kThreads - kWave) {
    const int upt = K * P.ng_routed + (L.has_shared ? P.ng_shared : 0);
    last_reader = arrive(tl + (1 + kFan) * kLine, upt + c, upt + P.nc);
  }
  float* hs = smem;                            // [S][Imax]
  float* hsum = hs + (size_t)P.S * P.Imax;     // [S][Imax/kCpc]
  uint16_t* sbl = reinterpret_cast<uint16_t*>(hsum + pad4(P.S * P.Imax / 16));   // 16-byte aligned
  if constexpr (FUSED) {
    // h arrives element by element with its "written" marks: once this
    // unit's own loads are in, poll the token's h (copy blockIdx % kHCopies
    // of the launch's buffer, one copy per XCD) until every element of every
    // slot is there
    drain();
    if (tid < n_sb) reinterpret_cast<uint4*>(sbl)[tid] = sbr;
    if (tid == 0) s_zx = zx;
    if (wid == 0 && L.has_shared && lane == K) {
      const uint32_t* sgp = P.sgb + s_par * kFusedMaxM + t;
      uint32_t v = 0;
      for (int i = 0; i < kSpinLimit && v == 0; ++i) {
        v = (uint32_t)ld_coh_i(reinterpret_cast<const int*>(sgp));
        if (v == 0) __builtin_amdgcn_s_sleep(8);
      }
      if (v == 0) atomicOr(P.ctr, 8);
      wk[K] = 1.0f / (1.0f + __expf(-__uint_as_float(~v)));
    }
    // first wait, cheaply, for one marker word per gate/up unit (the first
    // of its rows; wave 0 alone), so that the whole of h is loaded once it is
    // almost surely complete: polling all of it would put one copy of h per
    // poll round and down unit on the memory system while the weights stream
    const uint32_t* hw = P.hb + (size_t)s_par * P.hreg +
                         (size_t)(blockIdx.x % kHCopies) * P.P * P.Imax + (size_t)t * P.S * P.Imax;
    if (wid == 0) {
      const int nmk = K * P.ng_routed + P.ng_shared;
      constexpr int kMk = 8;
      for (int b0 = 0; b0 < nmk; b0 += kWave * kMk) {
        uint32_t need = 0;
#pragma unroll
        for (int j = 0; j < kMk; ++j)
          if (b0 + lane + kWave * j < nmk) need |= 1u << j;
        for (int spin = 0; spin < kSpinLimit; ++spin) {
          uint32_t v[kMk];
#pragma unroll
          for (int j = 0; j < kMk; ++j) {
            const int q = min(b0 + lane + kWave * j, nmk - 1);
            const int k = q < K * P.ng_routed ? q / P.ng_routed : K;
            const int g = k < K ? q - k * P.ng_routed : q - K * P.ng_routed;
            v[j] = (need >> j) & 1u ? (uint32_t)ld_coh_i(reinterpret_cast<const int*>(hw) + k * P.Imax + g * kGRows) : 0u;
          }
#pragma unroll
          for (int j = 0; j < kMk; ++j)
            if (v[j] != 0u) need &= ~(1u << j);
          if (__all(need == 0u)) break;
          __builtin_amdgcn_s_sleep(4);
        }
      }
    }
    __syncthreads();
    const uint64_t* h2 = reinterpret_cast<const uint64_t*>(hw);
    const int n2 = P.S * P.Imax / 2;
    constexpr int kB = 6;
    for (int b0 = 0; b0 < n2; b0 += kThreads * kB) {
      uint32_t need = 0;                       // bit j: item j of this batch still missing
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        const int i = b0 + tid + kThreads * j;
        if (i < n2) {
          const int k = (2 * i) / P.Imax;
          const int e = 2 * i - k * P.Imax;
          if (e < (k == K ? Is : I)) need |= 1u << j;
        }
      }
      for (int spin = 0; need && spin < kSpinLimit; ++spin) {
        // The first pass reads through the XCD's L2: every down unit that
        // reads this copy of h runs on the same XCD (workgroups are dealt to
        // the 8 XCDs round robin and the copy is picked by block index), so
        // one of them fetches a line from memory and the rest hit L2.  A line cached in L2 is never older than this launch (the L2s
        // are invalidated at kernel start) and values are only trusted when
        // their "written" mark is set; anything still missing is re-read
        // with coherent loads, which always go to memory.
        uint64_t rg[kB];
#pragma unroll
        for (int j = 0; j < kB; ++j) {
          const uint64_t* a = h2 + min(b0 + tid + kThreads * j, n2 - 1);
          rg[j] = (need >> j) & 1u ? (spin == 0 ? *a : ld_coh64(a)) : 0ull;
        }
#pragma unroll
        for (int j = 0; j < kB; ++j) {
          const uint32_t lo = (uint32_t)rg[j], hi = (uint32_t)(rg[j] >> 32);
          if (((need >> j) & 1u) && lo != 0u && hi != 0u) {
            const int i = b0 + tid + kThreads * j;
            const int k = (2 * i) / P.Imax;
            const int e = 2 * i - k * P.Imax;
            const int nk = (k == K ? Is : I) / kCpc;
            float* dst = hs + (size_t)k * P.Imax + 4 * ilv<kCpc>(e / 4, nk) + e % 4;
            dst[0] = __uint_as_float(~lo);
            dst[1] = __uint_as_float(~hi);
            need &= ~(1u << j);
          }
        }
        if (need) __builtin_amdgcn_s_sleep(8);
      }
      if (need) atomicOr(P.ctr, 8);
    }
  } else {
  // wait for token t's h (and the routing weights, the shared gate)
  if (wid == 0) {
    if (lane == 0 && !wait_flag(ready_line(P, d % kRep, t))) atomicOr(P.ctr, 1);
    // lane K: the shared expert's gate
    if (L.has_shared && lane == K) wk[K] = 1.0f / (1.0f + __expf(-ld_coh(P.sg + t)));
  }
  __syncthreads();
  // this unit is done with the token's flags: count it; the last unit of
  // the token lowers them for the next launch (below)
  if (tid == 0) s_done = arrive(tl + (1 + kFan) * kLine, c, P.nc);
  if (tid < n_sb) reinterpret_cast<uint4*>(sbl)[tid] = sbr;
  {
    // all coherent loads of a batch in flight before any is consumed
    const uint64_t* h2 = reinterpret_cast<const uint64_t*>(P.h + (size_t)(d % kHCopies) * P.P * P.Imax +
                                                           (size_t)t * P.S * P.Imax);
    const int n2 = P.S * P.Imax / 2;
    constexpr int kB = 8;
    for (int b0 = 0; b0 < n2; b0 += kThreads * kB) {
      uint64_t rg[kB];
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        const int i = b0 + tid + kThreads * j;
        rg[j] = ld_coh64(h2 + min(i, n2 - 1));
      }
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        const int i = b0 + tid + kThreads * j;   // floats 2i, 2i+1 of the token's h
        if (i < n2) {
          const int k = (2 * i) / P.Imax;
          const int e = 2 * i - k * P.Imax;      // element within the slot
          const int nk = (k == K ? Is : I) / kCpc;
          if (e < nk * kCpc) {
            float* dst = hs + (size_t)k * P.Imax + 4 * ilv<kCpc>(e / 4, nk) + e % 4;
            *reinterpret_cast<uint64_t*>(dst) = rg[j];
          }
        }
      }
    }
  }
  }
  if (FUSED && tid == kThreads - kWave) s_done = last_reader;
  __syncthreads();
  if (s_done) {
    if constexpr (FUSED) {
      for (int i = tid; i < kRep * K; i += kThreads) st_coh_u64(route_line(P, i / K, t) + i % K, 0);
    } else {
      if (tid < kRep) st_coh_i(ready_line(P, tid, t), 0);
    }
  }
  // chunk sums of every slot, one (slot, chunk) pair per thread
  for (int q = tid; q < tot; q += kThreads) {
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
  // the wave's row: per-lane partials over the lane's chunks, then the wave sum
  float pv[1];
  {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < DCH; ++j) {
      const int k = (kc[j] >> 16) - 1, cj = kc[j] & 0xFFFF;
      if (k >= 0 && rl < nrows) {
        const bool sh = k == K;
        const int Ik = sh ? Is : I;
        const int gpr = Ik >> esh;
        const float4* hk = reinterpret_cast<const float4*>(hs + (size_t)k * P.Imax);
        const float dd = chunk_dot<BITS>(wv[j], hk + cj, Ik / kCpc);
        const int gi = (sh ? K * kDRows * gr : k * kDRows * gr) + rl * gpr + ((cj * kCpc) >> esh);
        const int boff = K * kDRows * gr + kDRows * gs;    // biases follow all scales
        const float part = fmaf(bf16_to_f32(sbl[gi]), dd,
                                bf16_to_f32(sbl[boff + gi]) * hsum[(size_t)k * (P.Imax / kCpc) + cj]);
        acc = fmaf(wk[k], part, acc);
      }
    }
    pv[0] = acc;
  }
  const float tsum = treduce<1, 32>(pv, lane);
  if (lane == 0 && rl < nrows) {
    float v = bad ? __builtin_nanf("") : tsum;
    if (residual) v += resv;
    y[(size_t)t * H + r0 + rl] = v;
  }
  if constexpr (FUSED) {
    // clear this unit's share of the other parity's h and shared-gate
    // buffers: the previous launch used them (as much of the h buffer as its
    // extent word says, whatever its M), the next one fills them (off the
    // critical path, at the end)
    const size_t nh4 = min((size_t)(unsigned)s_zx, P.hreg / 4);
    const size_t per = (nh4 + (size_t)P.M * P.nc - 1) / ((size_t)P.M * P.nc);
    uint4* hz = reinterpret_cast<uint4*>(P.hb + (size_t)(s_par ^ 1) * P.hreg);
    for (size_t i = (size_t)d * per + tid; i < min(nh4, (size_t)(d + 1) * per); i += kThreads)
      hz[i] = make_uint4(0, 0, 0, 0);
    if (d == 0 && tid < kFusedMaxM) P.sgb[(s_par ^ 1) * kFusedMaxM + tid] = 0u;
  }
}

// 8-bit layers of up to 2048 columns: at most 80 VGPRs, so three units fit per
// CU (24 waves) and a 30B-A3B-shaped layer's units are all resident at once
template <int BITS, int CPL, int DCH, bool FUSED, bool NORM>
__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(BITS == 8 && CPL <= 2 && DCH <= 6 ? 6 : 1))) k_moe_decode(DecodeLayer L, DecPlan P, RouteIn R,
                                                        const float* __restrict__ x,
                                                        const int32_t* __restrict__ idx,
                                                        const float* __restrict__ wts,
                                                        const float* __restrict__ residual,
                                                        float* __restrict__ y) {
  int u = blockIdx.x;
  if constexpr (FUSED) {
    if (u < P.r_units) {
      route_unit<!(BITS == 8 && CPL <= 2 && DCH <= 6), NORM>(L, P, R, x, u);
      return;
    }
    u -= P.r_units;
  }
  if (u < P.g_units) gate_up_unit<BITS, CPL, FUSED, NORM>(L, P, x, idx, u);
  else down_unit<BITS, DCH, FUSED>(L, P, idx, wts, residual, y, u - P.g_units);
}

// The error word (the state block's first int, where every bounded wait of
// the decode launches records a timeout) out to the caller, then cleared.
__global__ void k_ws_status(int* word, int32_t* out, int timeout_status) {
  const int v = ld_coh_i(word);
  out[0] = v ? timeout_status : 0;
  out[1] = v;
  st_coh_i(word, 0);
}

int launch_ws_status(void* ws, int32_t* out, int timeout_status, hipStream_t s) {
  hipLaunchKernelGGL(k_ws_status, dim3(1), dim3(1), 0, s, reinterpret_cast<int*>(ws), out,
                     timeout_status);
  return 0;
}

DecState dec_state(const DecodeLayer& L, int K, void* ws) {
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  DecState D{};
  size_t off = 0;
  char* base = reinterpret_cast<char*>(ws);
  auto take = [&](size_t n) { char* p = base ? base + off : nullptr; off += al(n); return p; };
  const int S = K + (L.has_shared ? 1 : 0);
  const int Imax = L.has_shared && L.Is > L.I ? L.Is : L.I;
  D.ctr = reinterpret_cast<int*>(take(sizeof(int) * (size_t)kLine * (1 + (size_t)kCtrLines * kDecMaxM)));
  // flag copies: kRep blocks of kDecMaxM lines, 4 KB + 256 B apart at least
  D.rstride = (int)((((size_t)kDecMaxM * kLine * sizeof(int) + 4095) / 4096 * 4096 + 256) / sizeof(int));
  D.ready = reinterpret_cast<int*>(take(sizeof(int) * (size_t)kRep * D.rstride));
  D.epoch = reinterpret_cast<int*>(take(sizeof(int) * 4));
  D.hext = D.epoch ? D.epoch + 1 : nullptr;
  D.hreg = (size_t)kHCopies * kFusedMaxM * S * Imax;
  D.hb = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 2 * D.hreg));
  D.sgb = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 2 * kFusedMaxM));
  D.logits = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * (size_t)kFusedMaxM * L.E));
  D.idx_c = reinterpret_cast<int32_t*>(take(sizeof(int) * (size_t)kRep * D.rstride));
  D.route_ctr = reinterpret_cast<int*>(take(route_ctr_bytes()));
  D.bcounts = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)L.E));
  D.bytes = off;
  return D;
}

// the state block, then the launch's own data (h and the shared-gate logits
// of the launch without routing); M <= kDecMaxM
static DecPlan make_dec_plan(const DecodeLayer& L, int M, int K, bool routed, void* ws, size_t* bytes) {
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
  P.r_units = routed ? (L.E + kRRows - 1) / kRRows : 0;
  const DecState D = dec_state(L, K, ws);
  P.ctr = D.ctr;
  P.ready = D.ready;
  P.rstride = D.rstride;
  P.epoch = D.epoch;
  P.hext = D.hext;
  P.hb = D.hb;
  P.hreg = D.hreg;
  P.sgb = D.sgb;
  P.logits = D.logits;
  P.idx_c = D.idx_c;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  size_t off = D.bytes;
  char* base = reinterpret_cast<char*>(ws);
  auto take = [&](size_t n) { char* p = base ? base + off : nullptr; off += al(n); return p; };
  if (!routed) {
    P.h = reinterpret_cast<float*>(take(sizeof(float) * kHCopies * (size_t)P.P * P.Imax));
    P.sg = reinterpret_cast<float*>(take(sizeof(float) * (size_t)M));
  }
  if (bytes) *bytes = off;
  return P;
}

size_t decode_ws_bytes(const DecodeLayer& L, int M, int K, bool routed) {
  size_t b = 0;
  make_dec_plan(L, M, K, routed, nullptr, &b);
  return b;
}

// scale/bias words (16 bytes) a D unit stages: all slots, scales and biases
static int d_sb_words(const DecodeLayer& L, int K) {
  const int egs = L.gate.group_size;
  return 2 * kDRows * (K * (L.I / egs) + (L.has_shared ? L.Is / egs : 0)) * 2 / 16;
}

static size_t dec_lds_bytes(const DecodeLayer& L, int K, bool routed, int M) {
  // G: x (H floats) + chunk sums (<= H/16) + 4 x 16 rows x groups bf16;
  // D: h of all S slots (S x Imax floats) + their chunk sums (<= 1/16 of that)
  //    + the staged scale/bias words;
  // R (last unit only): E keys and E fp64 logits
  const size_t g = sizeof(float) * (L.H + pad4(L.H / 16)) + 2 * 4 * kGRows * (L.H / L.gate.group_size);
  const int S = K + (L.has_shared ? 1 : 0);
  const int Im = L.has_shared && L.Is > L.I ? L.Is : L.I;
  const size_t d = sizeof(float) * ((size_t)S * Im + pad4(S * Im / 16)) + 16 * (size_t)d_sb_words(L, K);
  const size_t r = routed ? 16 * (size_t)L.E : 0;        // + x of the M tokens below
  const size_t rx = routed ? sizeof(float) * (size_t)M * L.H : 0;
  size_t m = g > d ? g : d;
  m = m > r ? m : r;
  return m > rx ? m : rx;
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

// limits of this kernel: x at most 4096 floats (two 16-byte words per
// thread), G rows of at most 4 chunks per lane, D rows (all slots) of at most
// 8 chunks per lane, the shared expert at the routed experts' bit width, the
// scale/bias words of a G or D unit within one 16-byte word per thread, and
// the LDS
bool decode_supported(const DecodeLayer& L, int K) {
  const int b = L.gate.bits;
  if (L.H > 4096 || !g_cpl(L.H, b)) return false;
  if (4 * kGRows * (L.H / L.gate.group_size) * 2 / 16 > kThreads) return false;
  if (L.has_shared) {
    if (L.sh_gate.bits != b) return false;
    if (L.sh_eg.bits != 2 && L.sh_eg.bits != 4 && L.sh_eg.bits != 8) return false;
  }
  if (!d_ch(L, K)) return false;
  if (d_sb_words(L, K) > kThreads) return false;
  return dec_lds_bytes(L, K, false, 1) <= 160 * 1024;
}

bool fused_supported(const DecodeLayer& L, const QT& router, int M, int K) {
  return decode_supported(L, K) && router.bits == 8 && router.rows == L.E && router.cols == L.H &&
         M >= 1 && M <= kFusedMaxM && L.E <= kMaxExperts && dec_lds_bytes(L, K, true, M) <= 160 * 1024;
}

template <int B, int CPL, int DCH, bool FUSED, bool NORM>
static void run_dec(const DecodeLayer& L, const DecPlan& P, const RouteIn& R, const float* x,
                    const int32_t* idx, const float* w, const float* residual, float* y,
                    hipStream_t s) {
  const size_t lds = dec_lds_bytes(L, P.K, FUSED, P.M);
  hipLaunchKernelGGL((k_moe_decode<B, CPL, DCH, FUSED, NORM>), dim3(P.r_units + P.g_units + P.d_units),
                     dim3(kThreads), lds, s, L, P, R, x, idx, w, residual, y);
}

template <bool FUSED, bool NORM = false>
static int dispatch_dec(const DecodeLayer& L, const DecPlan& P, const RouteIn& R, const float* x,
                        const int32_t* idx, const float* w, const float* residual, float* y,
                        hipStream_t s) {
  const int b = L.gate.bits;
  const int cpl = g_cpl(L.H, b);
  const int dch = d_ch(L, P.K);
#define MOEQ_DEC(B_, C_, D_)                                              \
  if (b == B_ && cpl == C_ && dch == D_) {                               \
    run_dec<B_, C_, D_, FUSED, NORM>(L, P, R, x, idx, w, residual, y, s); \
    return 0;                                                            \
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

int launch_decode_forward(const DecodeLayer& L, const float* x, const int32_t* idx, const float* w,
                          int M, int K, const float* residual, float* y, void* ws, hipStream_t s) {
  if (M > kDecMaxM) return -9;
  const DecPlan P = make_dec_plan(L, M, K, false, ws, nullptr);
  const RouteIn R{};
  return dispatch_dec<false>(L, P, R, x, idx, w, residual, y, s);
}

int launch_moe_forward(const DecodeLayer& L, const RouteIn& R, const float* x, int M, int K,
                       const float* residual, float* y, void* ws, hipStream_t s) {
  if (M > kFusedMaxM) return -9;
  const DecPlan P = make_dec_plan(L, M, K, true, ws, nullptr);
  return dispatch_dec<true>(L, P, R, x, nullptr, nullptr, residual, y, s);
}

// the same launch with RMSNorm in front (router and experts see
// x / sqrt(mean(x^2) + eps) * g) and x added back in the combine
int launch_moe_forward_norm(const DecodeLayer& L, const RouteIn& R, const float* x, int M, int K,
                            const float* norm_w, float eps, float* y, void* ws, hipStream_t s) {
  if (M > kFusedMaxM) return -9;
  DecPlan P = make_dec_plan(L, M, K, true, ws, nullptr);
  P.norm_w = norm_w;
  P.norm_eps = eps;
  return dispatch_dec<true, true>(L, P, R, x, nullptr, nullptr, x, y, s);
}

}  // namespace moeq
