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
constexpr int kDRows = kWaves;             // output rows per D unit (one per wave), or 2 kDRows
                                           // when the layer's units outnumber the resident blocks
constexpr int kRRows = kWaves / 2;         // router rows per R unit (two waves per row)
constexpr int kSpinLimit = 1 << 26;
constexpr int kCUs = 256;                  // compute units of the chip (MI355X)
constexpr int kLine = kLineInts;
constexpr int kRep = 64;      // copies of every flag that many units poll
constexpr int kLogitCopies = 16;   // copies of the router logits (one per polling group of units)
static_assert(kLogitCopies % (kWave / kRRows) == 0,
              "a router unit writes its rows' logits to kWave / kRRows copies per store instruction");
constexpr int kSelCopies = 16;     // copies of the (expert, weight) pairs the down units poll
constexpr int kSelLine = 16;       // u64 words from one slot's pair to the next (a 128-byte line each)
// per token: G arrival counter lines, D arrival counter lines
constexpr int kCtrLines = 2 * (1 + kFan);
constexpr int kHCopies = 4;   // copies of h (down unit d reads copy d % kHCopies): spreads the reads of
                              // all D units of a token over more memory channels
static_assert(kHCopies * kGRows % kWave == 0, "a G unit's h copies are written by whole waves");
// the one-launch form's h buffers: a G unit's kGRows values (one segment) at
// the front of a 128-byte line of their own, so no line holds two segments
constexpr int kSegStride = 32;
static_assert(kSegStride * 4 == 128 && kGRows <= kSegStride, "a segment fills at most one line");

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

// ---- per-unit timestamps of one launch (timeline build only) ---------------
// Built with MOEQ_TIMELINE, every unit's first thread records the constant
// 100 MHz clock at the steps of its protocol into LDS, and the unit writes
// them to g_tl[block][event] when it ends (a global store per mark would
// hold up the unit's next memory wait until the store is acknowledged).
// Counters add up in LDS and are added to g_tl.  The product build compiles
// these marks away.
#ifdef MOEQ_TIMELINE
constexpr int kTlBlocks = 4096, kTlEvents = 12;
__device__ uint64_t g_tl[kTlBlocks * kTlEvents];
__device__ __forceinline__ uint64_t* tl_lds() {
  __shared__ uint64_t s_tl[2 * kTlEvents];   // marks, then counters
  return s_tl;
}
__device__ __forceinline__ void tl_begin() {
  if (threadIdx.x < 2 * kTlEvents) tl_lds()[threadIdx.x] = 0ull;
  __syncthreads();
}
__device__ __forceinline__ void tl_mark(int ev) {
  // the clock is read at this point of the program (nothing is moved across it)
  __builtin_amdgcn_sched_barrier(0);
  const uint64_t t = (uint64_t)wall_clock64();
  __builtin_amdgcn_sched_barrier(0);
  if (threadIdx.x == 0) {
    tl_lds()[ev] = t;
    // with the start mark: which XCD runs the block (hardware register XCC_ID, bits 3:0)
    if (ev == 0) tl_lds()[kTlEvents - 1] = (uint64_t)__builtin_amdgcn_s_getreg((3 << 11) | 20);
  }
}
// add n to the block's counter in event slot ev
__device__ __forceinline__ void tl_count(int ev, int n) {
  if (n) atomicAdd(reinterpret_cast<unsigned long long*>(tl_lds() + kTlEvents + ev), (unsigned long long)n);
}
__device__ __forceinline__ void tl_end() {
  __syncthreads();
  if (threadIdx.x < kTlEvents && blockIdx.x < kTlBlocks) {
    const uint64_t* s_tl = tl_lds();
    uint64_t* g = g_tl + (size_t)blockIdx.x * kTlEvents + threadIdx.x;
    if (s_tl[threadIdx.x]) *g = s_tl[threadIdx.x];
    if (s_tl[kTlEvents + threadIdx.x]) atomicAdd(reinterpret_cast<unsigned long long*>(g),
                                                 (unsigned long long)s_tl[kTlEvents + threadIdx.x]);
  }
}
#else
__device__ __forceinline__ void tl_begin() {}
__device__ __forceinline__ void tl_mark(int) {}
__device__ __forceinline__ void tl_count(int, int) {}
__device__ __forceinline__ void tl_end() {}
#endif


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
// top-K of one token from keys/vals in LDS (E <= 1024), all threads of the
// block, into sel[0..K) (LDS) in rank order; with wts, also the weights in
// fp64: p[idx]/sum p[idx] (renorm, summed in slot order) or p[idx]/sum over
// all E (fixed order), p relative to the maximum, rounded once to fp32.
// Keys are unique (topk.h), so ranks are too.  Up to 128 keys, every key is
// ranked against all; above, selection in three short steps instead:
//   1. the keys fall into 64 groups of g = ceil(E/64) consecutive keys; lane
//      i of wave 0 takes the maximum of group i;
//   2. T = the K-th largest of the 64 group maxima.  Exactly K groups have a
//      maximum >= T, so at least K keys are >= T and every key of the top K
//      is >= T; a key >= T lies in one of those K groups, so at most K g
//      keys are (the candidates);
//   3. the candidates are ranked among themselves: every key above a
//      candidate is a candidate too, so that rank is the rank among all E.
__device__ __forceinline__ void route_pick(const uint64_t* keys, const double* vals, int E, int K,
                                           int renorm, int* sel, float* wts) {
  constexpr int kMaxCand = kMaxTopK * (kMaxExperts / kWave);
  __shared__ uint64_t gmax[kWave];
  __shared__ uint64_t cand[kMaxCand];
  __shared__ uint64_t s_thr;
  __shared__ int s_nc;
  __shared__ double ex[kMaxTopK];
  __shared__ double red[kWaves];
  __shared__ double s_tot;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  if (E <= kThreads / 4) {
    // up to 128 experts: every key ranked against all, four threads per key
    const int a = tid >> 2, part = tid & 3;
    const uint64_t ka = a < E ? keys[a] : 0ull;
    int rank = 0;
#pragma unroll 8
    for (int j = part; j < E; j += 4) rank += keys[j] > ka;
    rank += __builtin_amdgcn_mov_dpp(rank, 0xB1, 0xF, 0xF, false);
    rank += __builtin_amdgcn_mov_dpp(rank, 0x4E, 0xF, 0xF, false);
    if (part == 0 && a < E && rank < K) sel[rank] = a;
  } else {
  const int g = (E + kWave - 1) / kWave;
  if (wid == 0) {
    uint64_t m = 0ull;                   // 0 is below every key (an empty group)
    const int lo = lane * g, hi = min(E, lo + g);
    for (int e = lo; e < hi; ++e) m = keys[e] > m ? keys[e] : m;
    gmax[lane] = m;
    if (lane == 0) s_nc = 0;
  }
  __syncthreads();
  {
    // rank of group maximum c among the 64, eight threads per maximum (at
    // least K groups are non-empty, so the K-th largest is a key)
    const int c = tid >> 3, part = tid & 7;
    if (c < kWave) {
      const uint64_t kc = gmax[c];
      int r = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) r += gmax[part * 8 + j] > kc;
      r += __shfl_xor(r, 1);
      r += __shfl_xor(r, 2);
      r += __shfl_xor(r, 4);
      if (part == 0 && r == K - 1) s_thr = kc;
    }
  }
  __syncthreads();
  {
    const uint64_t thr = s_thr;
    for (int e = tid; e < E; e += kThreads) {
      const uint64_t k = keys[e];
      if (k >= thr) cand[atomicAdd(&s_nc, 1)] = k;
    }
  }
  __syncthreads();
  {
    // tpc threads per candidate (a power of two, nc * tpc <= kThreads)
    const int nc = s_nc;
    int tpc = kWave / 4;
    while (tpc > 1 && nc * tpc > kThreads) tpc >>= 1;
    const int c = tid / tpc, part = tid & (tpc - 1);
    const uint64_t kc = c < nc ? cand[c] : 0ull;
    int r = 0;
    for (int j = part; j < nc; j += tpc) r += cand[j] > kc;
    for (int o = 1; o < tpc; o <<= 1) r += __shfl_xor(r, o);
    if (part == 0 && c < nc && r < K) sel[r] = 1023 - (int)(kc & 0x3FFull);
  }
  }
  __syncthreads();
  if (!wts) return;
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
  if (tid < K) wts[tid] = (float)(ex[tid] / s_tot);
  __syncthreads();
}

// Wave 0 of a G unit: wait until every router logit of token t is
// published (complemented fp64 bits, 0 = not yet), then put the token's keys
// and logits in LDS; returns the polling rounds it took.  One round loads the
// whole row and waits for it, so no load is left in flight at the end (a
// load still in flight would stall the first later use of its registers by
// a loaded memory latency).  Bounded: on the spin limit the error word gets
// bit 4 and the logits read as they are.
// kPer: logits per lane at most (E <= 64 kPer); kSleep: s_sleep between rounds
template <int kPer, int kSleep>
__device__ __forceinline__ int poll_logits(const uint64_t* lg, int E, int lane, int* err,
                                          uint64_t* keys, double* vals) {
  const int per = (E + kWave - 1) / kWave;
  uint64_t cur[kPer];
  int spin = 0;
  for (;; ++spin) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) cur[i] = i < per ? ld_coh_u64(lg + min(lane + kWave * i, E - 1)) : 1ull;
    bool all = true;
#pragma unroll
    for (int i = 0; i < kPer; ++i) all = all && cur[i] != 0ull;
    if (__all(all)) break;
    if (spin >= kSpinLimit) {
      if (lane == 0) atomicOr(err, 4);
      break;
    }
    __builtin_amdgcn_s_sleep(kSleep);
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + kWave * i;
    if (i < per && e < E) {
      const double v = __longlong_as_double((long long)~cur[i]);
      vals[e] = v;
      keys[e] = route_key(v, e);
    }
  }
  return spin;
}

// Router rows (8-bit) against x for all M tokens in fp64: the fp32
// dequantized weight widened exactly, fp64 products and sums, as the oracle
// defines the logits.  An R unit takes kRRows rows, two waves per row (wave
// half h takes the row's chunks lane + 64 (2j + h)), and publishes each
// finished logit into the launch's logits buffer; every G unit then selects
// its token's top-K itself (the D units take the slots' pairs from the G
// units).
// NORM: the rows see h = r * (x . g) with r = 1/sqrt(mean(x^2) + eps) per token
// (RMSNorm): x . g is staged, each token's mean square reduced over the block,
// and r applied to the finished logit.
template <bool NORM, int RCPL2>
__device__ __forceinline__ void route_unit(const DecodeLayer L, const DecPlan P, const RouteIn R,
                                           const float* __restrict__ x, int u) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int E = L.E, H = L.H, M = P.M;
  const int e = u * kRRows + wid / 2, h = wid & 1;
  tl_mark(0);                             // R: start
  const int nch = H / 16;                 // 16 codes per chunk at 8 bits (nch <= 128 RCPL2)
  const int rsh = __builtin_ctz((unsigned)R.W.group_size);   // log2 of the group size
  const int gpr = H >> rsh;
  __shared__ double part[kFusedMaxM][kRRows];
  const int er = min(e, E - 1);
  // the launch's parity picks its logits buffer (read now, so the load
  // overlaps the router rows)
  const int epoch = ld_coh_i(P.epoch);
  // Loads use clamped, always valid addresses and no branches, so they all
  // issue back to back; chunks past the row's end are never used.
  uint4 rv[RCPL2];
  uint32_t rsb[RCPL2];
#pragma unroll
  for (int j = 0; j < RCPL2; ++j) {
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
  __syncthreads();
  tl_mark(5);                             // R: router rows and x in
  double acc[kFusedMaxM];
#pragma unroll
  for (int m = 0; m < kFusedMaxM; ++m) acc[m] = 0.0;
  if (M == 1) {
    // one token: the chunk's 16 activations are read from LDS together and
    // the chunk keeps four independent fp64 chains (one per 4-code word)
#pragma unroll
    for (int j = 0; j < RCPL2; ++j) {
      const int c = lane + kWave * (2 * j + h);
      const int cc = min(c, nch - 1);
      const float rs = bf16_to_f32(rsb[j] & 0xFFFFu), rb = bf16_to_f32(rsb[j] >> 16);
      float4 xv[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) xv[f] = xl[f * nch + cc];
      double a[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const uint32_t wd = f == 0 ? rv[j].x : f == 1 ? rv[j].y : f == 2 ? rv[j].z : rv[j].w;
        double t = (double)fmaf(rs, (float)(wd & 0xFFu), rb) * (double)xv[f].x;
        t = fma((double)fmaf(rs, (float)((wd >> 8) & 0xFFu), rb), (double)xv[f].y, t);
        t = fma((double)fmaf(rs, (float)((wd >> 16) & 0xFFu), rb), (double)xv[f].z, t);
        a[f] = fma((double)fmaf(rs, (float)(wd >> 24), rb), (double)xv[f].w, t);
      }
      if (c < nch) acc[0] += (a[0] + a[1]) + (a[2] + a[3]);
    }
  } else {
    // per lane and token, its chunks as independent fp64 chains, elements in
    // order; a weight is dequantized once for all tokens; one chunk at a time
    // (the scheduling barrier keeps the compiler from hoisting every chunk's
    // fp64 operands at once)
#pragma unroll
    for (int j = 0; j < RCPL2; ++j) {
      const int c = lane + kWave * (2 * j + h);
      if (c < nch) {
        const float rs = bf16_to_f32(rsb[j] & 0xFFFFu), rb = bf16_to_f32(rsb[j] >> 16);
        const uint32_t wd[4] = {rv[j].x, rv[j].y, rv[j].z, rv[j].w};
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          double w[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) w[q] = (double)fmaf(rs, (float)((wd[f] >> (8 * q)) & 0xFFu), rb);
#pragma unroll
          for (int m = 0; m < kFusedMaxM; ++m) {
            if (m < M) {
              const float4 xv = xl[m * (H / 4) + f * nch + c];
              acc[m] = fma(w[0], (double)xv.x, acc[m]);
              acc[m] = fma(w[1], (double)xv.y, acc[m]);
              acc[m] = fma(w[2], (double)xv.z, acc[m]);
              acc[m] = fma(w[3], (double)xv.w, acc[m]);
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  tl_mark(1);                             // R: fp64 dot products done
  // the two halves of a row meet in LDS; the even wave publishes the logit
  double wsum[kFusedMaxM];
#pragma unroll
  for (int m = 0; m < kFusedMaxM; ++m) {
    wsum[m] = 0.0;
    if (m < M) {
      wsum[m] = wave_sum_d(acc[m]);
      if (h == 1 && lane == 0) part[m][wid / 2] = wsum[m];
    }
  }
  __syncthreads();
  // every logit goes to kLogitCopies copies, one per lane (a G unit
  // polls copy blockIdx % kLogitCopies: many units polling one line would
  // queue on its memory channel)
  // the unit's kRRows logits of a token are staged, then written to every
  // copy as one run of kRRows consecutive values: adjacent lanes take the
  // rows of one copy, so each copy's run is one coalesced write
  __shared__ uint64_t s_pub[kFusedMaxM][kRRows];
#pragma unroll
  for (int m = 0; m < kFusedMaxM; ++m) {
    if (m < M && h == 0 && lane == 0) {
      double tot = wsum[m] + part[m][wid / 2];
      if constexpr (NORM) {
        float sq = 0.f;
        for (int w = 0; w < kWaves; ++w) sq += s_ss[w][m];
        tot *= 1.0 / sqrt((double)sq / H + (double)P.norm_eps);
      }
      // published as the complement of its bits: zero means "not written
      // yet" (the complement of a finite double is never zero)
      s_pub[m][wid / 2] = ~(uint64_t)__double_as_longlong(tot);
    }
  }
  __syncthreads();
  if (wid == 0) {
    const int r = lane % kRRows, e0 = u * kRRows;
    constexpr int kCpI = kWave / kRRows;           // copies per store instruction
#pragma unroll
    for (int j = 0; j < kLogitCopies / kCpI; ++j) {
      const int c = lane / kRRows + kCpI * j;
      uint64_t* lg = P.logits + ((size_t)(epoch & 1) * kLogitCopies + c) * P.lstride;
#pragma unroll
      for (int m = 0; m < kFusedMaxM; ++m)
        if (m < M && e0 + r < E) st_coh_u64(lg + (size_t)m * E + e0 + r, s_pub[m][r]);
    }
  }
  tl_mark(2);                             // R: logits published
}

// ------------------------------------------------------------------ G unit
// LDS: [x, chunk-interleaved][its chunk sums (<= H/16 floats)][bf16 scales and
// biases of the unit's gate and up rows]
template <int BITS, int CPL, bool FUSED, bool NORM, bool WIDE, int POLL>
__device__ __forceinline__ void gate_up_unit(const DecodeLayer L, const DecPlan P,
                                             const float* __restrict__ x,
                                             const int32_t* __restrict__ idx, int u, int renorm) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ int s_done;
  __shared__ int s_sel[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
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
  tl_mark(0);                                       // G: start
  // the launch's parity (its logits and h buffers), read first
  const int par = FUSED ? (ld_coh_i(P.epoch) & 1) : 0;
  float* xs = smem;
  float* xsum = xs + H;
  // (the sums' region is padded to 16 bytes: the scale words are stored as uint4)
  uint16_t* sbl = reinterpret_cast<uint16_t*>(xsum + pad4(H / 16));   // [4][kGRows * gpr]
  float4* x4 = reinterpret_cast<float4*>(xs);
  // the token's router keys and logits while it selects (after the scales)
  uint64_t* keys = reinterpret_cast<uint64_t*>(sbl + 4 * kGRows * gpr);
  double* vals = reinterpret_cast<double*>(keys + L.E);

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
    tl_mark(1);                                     // G: x staged
    if (!shared) {
      // the token's top-K from the published logits; this unit's expert is
      // the one in its slot
      if (wid == 0) {
        const int rounds =
            poll_logits<POLL, 1>(P.logits + ((size_t)par * kLogitCopies + blockIdx.x % kLogitCopies) * P.lstride +
                                  (size_t)t * L.E,
                              L.E, lane, P.ctr, keys, vals);
        tl_mark(5);                                 // G: logits seen
        if (lane == 0) tl_count(6, rounds + 1);
      }
      __syncthreads();
      tl_mark(7);                                   // G: after the barrier
      // the slot's first unit also takes the routing weights and publishes
      // the slot's (expert, weight) pair for the down units, in every copy
      route_pick(keys, vals, L.E, K, g == 0 ? renorm : 0, s_sel, g == 0 ? s_w : nullptr);
      if (g == 0 && wid == 0 && lane < kSelCopies)
        st_coh_u64(P.selw + ((size_t)par * kSelCopies + lane) * P.sstride + ((size_t)t * kMaxTopK + k) * kSelLine,
                   ~(((uint64_t)(uint32_t)s_sel[k] << 32) | __float_as_uint(s_w[k])));
    }
    tl_mark(2);                                     // G: expert known
    if (!shared) erow = (size_t)min(max(s_sel[k], 0), L.E - 1) * L.I;
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
  tl_mark(3);                                       // G: weights in, partial dots done
  const float gsum = treduce<2, 32>(pg, lane);
  const float usum = treduce<2, 32>(pu, lane);
  float rn = 1.f;
  if constexpr (NORM) {
    float sq = 0.f;
    for (int w = 0; w < kWaves; ++w) sq += s_gss[w];
    rn = (float)(1.0 / sqrt((double)sq / H + (double)P.norm_eps));
  }
  if constexpr (FUSED) {
    // the unit's rows meet in LDS, then one wave writes every copy, the
    // kGRows values of a copy (one 64-byte segment) by one store instruction,
    // as complemented bits (0 means "not written in this launch"): a down unit
    // that sees a segment's first value sees the rest of it too, as a rule
    __shared__ float s_h[kGRows];
    if ((lane & 31) == 0) {               // every lane of a half holds its row's sum
      const int i = wid * 2 + tindex<2, 32>(lane);
      s_h[i] = valid ? silu(rn * gsum) * (rn * usum) : __builtin_nanf("");
    }
    __syncthreads();
    if (wid == 0) {
#pragma unroll
      for (int j = 0; j < kHCopies * kGRows / kWave; ++j) {
        const int q = lane + kWave * j, c = q / kGRows, i = q % kGRows;
        if (i < nrows)
          st_coh_i(reinterpret_cast<int*>(P.hb) + (size_t)par * P.hreg + (size_t)c * P.P * P.hstride +
                       (size_t)p * P.hstride + g * kSegStride + i,
                   (int)~__float_as_uint(s_h[i]));
      }
    }
  } else if ((lane & 31) < kHCopies) {  // every lane of a half holds its row's sum
    const int i = wid * 2 + tindex<2, 32>(lane);
    const float hv = valid ? silu(rn * gsum) * (rn * usum) : __builtin_nanf("");
    if (i < nrows)
      st_coh(P.h + (size_t)(lane & 31) * P.P * P.Imax + (size_t)p * P.Imax + i_base + i, hv);
  }
  tl_mark(4);                                       // G: h written
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
        st_coh_i(reinterpret_cast<int*>(P.sgb) + par * kFusedMaxM + t, (int)~__float_as_uint(tot));
      else
        st_coh(P.sg + t, tot);
    }
  }
  if constexpr (!FUSED) {
    // h goes out with the ready flag (the one-launch form's h carries its own
    // "written" marks instead)
    drain();
    __syncthreads();
    if (tid == 0) s_done = arrive(P.ctr + (size_t)kLine * (1 + (size_t)t * kCtrLines), r, upt);
    __syncthreads();
    if (s_done && tid < kRep) st_coh_i(ready_line(P, tid, t), 1);
  }
}

// scale/bias words (16 bytes) a D unit stages: all slots, scales and biases
__host__ __device__ __forceinline__ int d_sb_words_dev(const DecodeLayer& L, int K, int dr) {
  const int egs = L.gate.group_size;
  return 2 * dr * (K * (L.I / egs) + (L.has_shared ? L.Is / egs : 0)) * 2 / 16;
}

// ------------------------------------------------------------------ D unit
// LDS: [h of all S slots, chunk-interleaved per slot][their chunk sums][bf16
// scales then biases of the unit's rows, slot by slot]
template <int BITS, int DCH, int DR, bool FUSED, bool WIDE, int POLL>
__device__ __forceinline__ void down_unit(const DecodeLayer L, const DecPlan P, const RouteIn R,
                                          const int32_t* __restrict__ idx,
                                          const float* __restrict__ wts,
                                          const float* __restrict__ residual,
                                          float* __restrict__ y, int d) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ float wk[kMaxTopK + 1];
  __shared__ int s_ex[kMaxTopK];
  __shared__ int bad, s_done, s_zx, s_late;
  constexpr int kCpc = 128 / BITS;
  // segments of a token a thread may own (DCH chunks per lane of kCpc values)
  constexpr int kSegPT = (DCH * kCpc + 127) / 128;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int K = P.K, H = L.H;
  const int t = d / P.nc;
  const int c = d - t * P.nc;
  const int r0 = c * DR;
  const int nrows = min(DR, H - r0);
  const int I = L.I, Is = L.Is;
  const int cpr = I / kCpc;                    // chunks per routed down row
  const int cps = L.has_shared ? Is / kCpc : 0;
  const int tot = K * cpr + cps;               // chunks per output row, all slots
  tl_mark(0);                                  // D: start
  // the launch's parity (its logits and h buffers), read first
  // (the fused form reads the launch's parity with its first poll below)
  int par = 0;
  int* tl = P.ctr + (size_t)kLine * (1 + (size_t)t * kCtrLines);
  // the thread's chunk and rows: the threads form kTG groups of kThreads/kTG
  // (kTG = 8/DCH rounded down to a power of two, so a group has a thread
  // for each of the tot <= 64 DCH chunks of all slots); group gq takes rows
  // gq kRPT ... + kRPT - 1, its thread lq chunk lq: slot kq (-1: none),
  // chunk cq within the slot
  constexpr int kTG = DCH == 1 ? 8 : DCH == 2 ? 4 : DCH <= 4 ? 2 : 1;
  constexpr int kRPT = DR / kTG;
  const int gq = tid / (kThreads / kTG), lq = tid % (kThreads / kTG);
  const int kq = lq < tot ? (lq < K * cpr ? lq / cpr : K) : -1;
  const int cq = kq < 0 ? 0 : (kq < K ? lq - kq * cpr : lq - K * cpr);

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
  // (the router keys and logits of the token in LDS while it selects, past
  // the unit's h, chunk sums and scale/bias words)
  float* hs = smem;                            // [S][Imax]
  // (then a region of S * Imax / 16 floats, unused, ahead of the scales)
  uint16_t* sbl = reinterpret_cast<uint16_t*>(hs + (size_t)P.S * P.Imax + pad4(P.S * P.Imax / 16));
  if constexpr (FUSED) {
    // the token's top-K and its weights: the (expert, weight) pair each
    // slot's first gate/up unit publishes; the token's first D unit also
    // writes them out for the caller.  The first round reads the launch
    // counter and both parities' pairs together and keeps the pairs of the
    // parity the counter names (those were cleared by the previous launch),
    // so a unit that starts late finds its pairs one memory round trip
    // earlier.
    __shared__ int s_par;
    if (wid == 0) {
      const size_t cp = blockIdx.x % kSelCopies;
      const uint64_t* sp0 = P.selw + cp * P.sstride + (size_t)t * kMaxTopK * kSelLine;
      const uint64_t* sp1 = P.selw + ((size_t)kSelCopies + cp) * P.sstride + (size_t)t * kMaxTopK * kSelLine;
      const int ep = ld_coh_i(P.epoch);
      const uint64_t v0 = lane < K ? ld_coh_u64(sp0 + lane * kSelLine) : 1ull;
      const uint64_t v1 = lane < K ? ld_coh_u64(sp1 + lane * kSelLine) : 1ull;
      const int pr = ep & 1;
      const uint64_t* sp = pr ? sp1 : sp0;
      uint64_t v = pr ? v1 : v0;
      int spin = 0;
      for (;; ++spin) {
        if (__all(v != 0ull)) break;
        if (spin >= kSpinLimit) {
          if (lane == 0) atomicOr(P.ctr, 4);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        v = lane < K ? ld_coh_u64(sp + lane * kSelLine) : 1ull;
      }
      // pairs already there at the first look: the unit started after the
      // gate/up units' first rows were done, and h is likely complete
      if (lane == 0) s_late = spin == 0;
      if (lane < K) {
        v = ~v;
        s_ex[lane] = (int)(uint32_t)(v >> 32);
        wk[lane] = __uint_as_float((uint32_t)v);
      }
      if (lane == 0) s_par = pr;
    }
    __syncthreads();
    par = s_par;
    if (tid < K) {
      if (c == 0) {
        R.idx_out[(size_t)t * K + tid] = s_ex[tid];
        R.w_out[(size_t)t * K + tid] = wk[tid];
      }
      s_ex[tid] = min(max(s_ex[tid], 0), L.E - 1);
    }
  }
  __syncthreads();
  tl_mark(1);                                  // D: experts known
  // scales and biases of every slot (per slot DR rows x groups bf16,
  // contiguous), then the routed chunks
  const int esh = __builtin_ctz((unsigned)L.gate.group_size);  // log2 group size, every expert matrix
  const int gr = I >> esh, gs = L.has_shared ? Is >> esh : 0;
  const int sb_r = DR * gr * 2 / 16;       // 16-byte words per slot and tensor
  const int sb_s = DR * gs * 2 / 16;
  const int n_sb = 2 * (K * sb_r + sb_s);      // all slots, scales and biases
  // (clamped, always valid addresses and no branches: the loads issue back
  // to back; H is a multiple of DR, so every unit has full rows)
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
  // the residual of the unit's rows goes out with its other loads, so the
  // final sum does not wait for it (threads tid < DR write the rows)
  float resv = 0.f;
  if (residual && tid < DR) resv = residual[(size_t)t * H + r0 + min(tid, nrows - 1)];
  // the thread's chunk of every row (a thread without a chunk reads a valid
  // one and never uses it)
  uint4 wr[kRPT];
  {
    const bool sh = kq == K;
    const uint32_t* base = sh ? L.sh_down.q
                              : L.down.q + ((size_t)s_ex[max(kq, 0)] * H) * (I / (32 / BITS));
    const int wpr = (sh ? Is : I) / (32 / BITS);
#pragma unroll
    for (int r = 0; r < kRPT; ++r)
      wr[r] = reinterpret_cast<const uint4*>(base + (size_t)(r0 + min(gq * kRPT + r, nrows - 1)) * wpr)[cq];
  }
  // the extent of the other h buffer's last use (cleared at the end)
  const int zx = FUSED ? ld_coh_i(P.hext + (par ^ 1)) : 0;
  if constexpr (FUSED) {
    // h arrives element by element with its "written" marks: once this
    // unit's own loads are in, poll the token's h (copy blockIdx % kHCopies
    // of the launch's buffer, one copy per XCD) until every element of every
    // slot is there
    drain();
    if (tid < n_sb) reinterpret_cast<uint4*>(sbl)[tid] = sbr;
    if (tid == 0) s_zx = zx;
    if (wid == 0 && L.has_shared && lane == K) {
      const uint32_t* sgp = P.sgb + par * kFusedMaxM + t;
      uint32_t v = 0;
      for (int i = 0; i < kSpinLimit && v == 0; ++i) {
        v = (uint32_t)ld_coh_i(reinterpret_cast<const int*>(sgp));
        if (v == 0) __builtin_amdgcn_s_sleep(8);
      }
      if (v == 0) atomicOr(P.ctr, 8);
      wk[K] = 1.0f / (1.0f + __expf(-__uint_as_float(~v)));
    }
    __syncthreads();                             // staged scales and biases, wk[K]
    // h arrives segment by segment: a G unit writes each copy of its kGRows
    // values (one segment, alone in a 128-byte line) with one store
    // instruction, as complemented bits (0 = not written).  Every thread
    // owns segments tid + kThreads i: it polls a segment's first value with a
    // coherent load and, one round later, loads the whole segment through
    // L2 into LDS (its line cannot be in L2 from before the segment was
    // whole: only a D unit that saw its first value reads it).  So h lands in
    // LDS while the gate/up units are still finishing, and after the last
    // one only its segment is left to fetch.  Values found unwritten are
    // re-read with coherent loads.
    const uint32_t* hw = P.hb + (size_t)par * P.hreg +
                         (size_t)(blockIdx.x % kHCopies) * P.P * P.hstride +
                         (size_t)t * P.S * P.hstride;
    const int nseg = K * P.ng_routed + P.ng_shared;   // segments of the token
    uint32_t pend = 0, seen = 0, slow = 0;       // this thread's segments q = tid + kThreads i
#pragma unroll
    for (int i = 0; i < kSegPT; ++i)
      if (tid + kThreads * i < nseg) pend |= 1u << i;
    // a unit that started late reads the segments whole in its first round
    // (no marker round first): a segment found incomplete that way is re-read
    // with coherent loads from then on, since its line may now sit in L2
    if (s_late) seen = pend;
    for (int round = 0;; ++round) {
      if (pend) {
        uint32_t mk[kSegPT];
        uint4 body[kSegPT][kGRows / 4];
#pragma unroll
        for (int i = 0; i < kSegPT; ++i) {
          const int q = min(tid + kThreads * i, nseg - 1);
          const int k = q < K * P.ng_routed ? q / P.ng_routed : K;
          const int g = k < K ? q - k * P.ng_routed : q - K * P.ng_routed;
          const uint32_t* src = hw + (size_t)k * P.hstride + g * kSegStride;
          mk[i] = 0u;
          if ((pend >> i) & 1u) {
            if (!((seen >> i) & 1u)) {
              mk[i] = (uint32_t)ld_coh_i(reinterpret_cast<const int*>(src));
            } else if (!((slow >> i) & 1u)) {
#pragma unroll
              for (int f = 0; f < kGRows / 4; ++f) body[i][f] = reinterpret_cast<const uint4*>(src)[f];
            } else {
#pragma unroll
              for (int f = 0; f < kGRows / 4; ++f) {
                const uint64_t a = ld_coh64(reinterpret_cast<const uint64_t*>(src) + 2 * f);
                const uint64_t b = ld_coh64(reinterpret_cast<const uint64_t*>(src) + 2 * f + 1);
                body[i][f] = make_uint4((uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32));
              }
            }
          }
        }
#pragma unroll
        for (int i = 0; i < kSegPT; ++i) {
          if (!((pend >> i) & 1u)) continue;
          if (!((seen >> i) & 1u)) {
            if (mk[i] != 0u) seen |= 1u << i;
            continue;
          }
          bool full = true;
#pragma unroll
          for (int f = 0; f < kGRows / 4; ++f)
            full = full && body[i][f].x != 0u && body[i][f].y != 0u && body[i][f].z != 0u && body[i][f].w != 0u;
          if (!full) {                           // a value not visible yet: re-read from memory
            if (!((slow >> i) & 1u)) tl_count(5, 1);
            slow |= 1u << i;
            continue;
          }
          const int q = tid + kThreads * i;
          const int k = q < K * P.ng_routed ? q / P.ng_routed : K;
          const int g = k < K ? q - k * P.ng_routed : q - K * P.ng_routed;
          const int nk = (k == K ? Is : I) / kCpc;
          float4* dst = reinterpret_cast<float4*>(hs + (size_t)k * P.Imax);
#pragma unroll
          for (int f = 0; f < kGRows / 4; ++f)
            dst[ilv<kCpc>(g * (kGRows / 4) + f, nk)] =
                make_float4(__uint_as_float(~body[i][f].x), __uint_as_float(~body[i][f].y),
                            __uint_as_float(~body[i][f].z), __uint_as_float(~body[i][f].w));
          pend &= ~(1u << i);
        }
      }
      if (__syncthreads_and(pend == 0u)) {
        tl_mark(2);                              // D: every segment of h in LDS
        if (tid == 0) tl_count(6, round + 1);    // rounds the unit took
        break;
      }
      if (round >= kSpinLimit / 64) {            // bounded: give up, record it
        if (tid == 0) atomicOr(P.ctr, 8);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
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
  if constexpr (!FUSED) {
    __syncthreads();
    if (s_done && tid < kRep) st_coh_i(ready_line(P, tid, t), 0);
  }
  tl_mark(3);                                  // D: h of every slot staged
  // every thread: its chunk of h read from LDS (and summed) and applied to
  // its chunk of its group's kRPT rows; the chunk's term per row is
  // w_k (s (codes . h) + b (sum of h)), s and b the row's group
  float part[kRPT];
#pragma unroll
  for (int r = 0; r < kRPT; ++r) part[r] = 0.f;
  if (kq >= 0) {
    const bool sh = kq == K;
    const int Ik = sh ? Is : I;
    const int gpr = Ik >> esh;
    const int nk = Ik / kCpc;
    const float4* hk = reinterpret_cast<const float4*>(hs + (size_t)kq * P.Imax);
    float dd[kRPT];
#pragma unroll
    for (int r = 0; r < kRPT; ++r) dd[r] = 0.f;
    // (codes converted in byte passes, as in chunk_dot)
    float hsm = 0.f;
    constexpr int kF = 8 / BITS, kPasses = 8 / BITS;
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
      float4 hv[kF];
#pragma unroll
      for (int f = 0; f < kF; ++f) {
        hv[f] = hk[(wi * kF + f) * nk + cq];
        hsm += (hv[f].x + hv[f].y) + (hv[f].z + hv[f].w);
      }
#pragma unroll
      for (int r = 0; r < kRPT; ++r) {
        const uint32_t w = wi == 0 ? wr[r].x : wi == 1 ? wr[r].y : wi == 2 ? wr[r].z : wr[r].w;
#pragma unroll
        for (int m = 0; m < kPasses; ++m) {
          const uint32_t t = code_pass<BITS>(w, m);
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int j = BITS == 2 ? 4 * b + m : BITS == 4 ? 2 * b + m : b;
            dd[r] = fmaf((float)((t >> (8 * b)) & 0xFFu), f4c(hv[j / 4], j % 4), dd[r]);
          }
        }
      }
    }
    const int g0 = (sh ? K * DR * gr : kq * DR * gr) + gq * kRPT * gpr + ((cq * kCpc) >> esh);
    const int boff = K * DR * gr + DR * gs;    // biases follow all scales
    const float wkq = wk[kq];
#pragma unroll
    for (int r = 0; r < kRPT; ++r)
      part[r] = wkq * fmaf(bf16_to_f32(sbl[g0 + r * gpr]), dd[r],
                           bf16_to_f32(sbl[boff + g0 + r * gpr]) * hsm);
  }
  // each row summed over the wave (one transposed reduction of the kRPT
  // values), then over its group's waves in order: a fixed order, so the
  // result does not change from run to run
  __shared__ float s_red[kWaves][kRPT];
  {
    const float v = treduce<kRPT, 32>(part, lane);
    if ((lane & (kWave / kRPT - 1)) == 0) s_red[wid][tindex<kRPT, 32>(lane)] = v;
  }
  __syncthreads();
  if (tid < nrows) {
    constexpr int kWG = kWaves / kTG;            // waves per group
    const int g = tid / kRPT, rr = tid % kRPT;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kWG; ++w) sum += s_red[g * kWG + w][rr];
    float v = bad ? __builtin_nanf("") : sum;
    if (residual) v += resv;
    y[(size_t)t * H + r0 + tid] = v;
  }
  tl_mark(4);                                  // D: y written
  if constexpr (FUSED) {
    // clear this unit's share of the other parity's h, logits, selection and
    // shared-gate buffers: the previous launch used them (as much of the h
    // buffer as its extent word says, whatever its M), the next one fills
    // them (off the critical path, at the end)
    const size_t nd = (size_t)P.M * P.nc;
    const size_t nh4 = min((size_t)(unsigned)s_zx, P.hreg / 4);
    const size_t per = (nh4 + nd - 1) / nd;
    uint4* hz = reinterpret_cast<uint4*>(P.hb + (size_t)(par ^ 1) * P.hreg);
    for (size_t i = (size_t)d * per + tid; i < min(nh4, (size_t)(d + 1) * per); i += kThreads)
      hz[i] = make_uint4(0, 0, 0, 0);
    const size_t nl = (size_t)kLogitCopies * P.lstride;
    const size_t perl = (nl + nd - 1) / nd;
    uint64_t* lz = P.logits + (size_t)(par ^ 1) * nl;
    for (size_t i = (size_t)d * perl + tid; i < min(nl, (size_t)(d + 1) * perl); i += kThreads) lz[i] = 0ull;
    const size_t ns = (size_t)kSelCopies * P.sstride;
    const size_t pers = (ns + nd - 1) / nd;
    uint64_t* sz = P.selw + (size_t)(par ^ 1) * ns;
    for (size_t i = (size_t)d * pers + tid; i < min(ns, (size_t)(d + 1) * pers); i += kThreads) sz[i] = 0ull;
    if (d == 0 && tid < kFusedMaxM) P.sgb[(par ^ 1) * kFusedMaxM + tid] = 0u;
    // how much of this launch's h buffer it fills (the launch after next
    // clears that much of it)
    if (d == 0 && tid == 0) st_coh_i(P.hext + par, (int)((size_t)kHCopies * P.P * P.hstride / 4));
    // the last D unit of the launch to get here moves the launch counter on:
    // every unit of this launch has read it by then (each D unit has, and
    // every G and R unit ran before the last D unit could finish)
    drain();
    __syncthreads();
    if (tid == 0 && arrive(P.dctr, d, (int)nd)) st_coh_i(P.epoch, ld_coh_i(P.epoch) + 1);
  }
}

// Block -> unit (0 R, 1 G, 2 D; *u its index among its kind).  With routing
// in the launch (r_half != 0) the R units take the first r_half positions on
// XCDs 0 and 1: workgroups are dealt to the XCDs round robin (block b to XCD
// b % 8) and the XCDs start dispatching one after another, XCD 0 first, so
// the router rows and the selector (R unit 0 = block 0) start earliest.  The
// other blocks, in order, are the G units, then the D units, so on every XCD
// the units a unit waits for come before it.
__device__ __forceinline__ int unit_of(int b, const DecPlan& P, int* u) {
  if (P.r_half) {
    const int q = b >> 3, xcd = b & 7;
    if (xcd < 2 && q < P.r_half) {
      *u = 2 * q + xcd;
      return 0;
    }
    b -= 2 * min(q, P.r_half) + (q < P.r_half ? min(xcd, 2) : 0);
  } else if (b < P.r_units) {
    *u = b;
    return 0;
  } else {
    b -= P.r_units;
  }
  if (b < P.g_units) {
    *u = b;
    return 1;
  }
  *u = b - P.g_units;
  return 2;
}

// 8-bit layers of up to 2048 columns: at most 80 VGPRs, so three units fit per
// CU (24 waves) and a 30B-A3B-shaped layer's units are all resident at once
template <int BITS, int CPL, int DCH, int DR, bool FUSED, bool NORM>
__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(BITS == 8 && CPL <= 2 && DCH <= 6 ? 6 : 1))) k_moe_decode(DecodeLayer L, DecPlan P, RouteIn R,
                                                        const float* __restrict__ x,
                                                        const int32_t* __restrict__ idx,
                                                        const float* __restrict__ wts,
                                                        const float* __restrict__ residual,
                                                        float* __restrict__ y) {
  // the 80-register form (8-bit, narrow rows) keeps the one-wave selection
  // and the logit polls small: E <= 256 there
  constexpr bool kWide = !(BITS == 8 && CPL <= 2 && DCH <= 6);
  constexpr int kPoll = kWide ? kMaxExperts / kWave : 4;
  int u;
  const int role = unit_of((int)blockIdx.x, P, &u);
  tl_begin();
  // router chunks per lane and wave half: H / 2048, from the G units' CPL
  constexpr int kRc = CPL * 4 / BITS < 1 ? 1 : (CPL * 4 / BITS > 2 ? 2 : CPL * 4 / BITS);
  if (FUSED && role == 0) route_unit<NORM, kRc>(L, P, R, x, u);
  else if (role == 1) gate_up_unit<BITS, CPL, FUSED, NORM, kWide, kPoll>(L, P, x, idx, u, R.renorm);
  else down_unit<BITS, DCH, DR, FUSED, kWide, kPoll>(L, P, R, idx, wts, residual, y, u);
  tl_end();
}

#ifdef MOEQ_TIMELINE
// timeline build only: the last launch's timestamps out to the host
extern "C" int moeq_timeline_copy(uint64_t* host, size_t n) {
  if (n > (size_t)kTlBlocks * kTlEvents) n = (size_t)kTlBlocks * kTlEvents;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_tl), n * sizeof(uint64_t)) == hipSuccess ? 0 : -10;
}
extern "C" int moeq_timeline_clear() {
  static uint64_t zeros[kTlBlocks * kTlEvents];
  return hipMemcpyToSymbol(HIP_SYMBOL(g_tl), zeros, sizeof(zeros)) == hipSuccess ? 0 : -10;
}

// The read ceiling the decode layer streams against: `bytes` read once in
// 16-byte loads, four in flight per thread, by `blocks` blocks of 256 threads
// (each block's words folded into one value, stored only if it is a
// sentinel, so the loads cannot be dropped).
__global__ void __launch_bounds__(256) k_read_probe(const uint4* __restrict__ p, size_t n16,
                                                    uint32_t* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * 256;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) out[blockIdx.x] = acc;
}

extern "C" int moeq_read_probe(const void* p, size_t bytes, int blocks, uint32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(k_read_probe, dim3(blocks), dim3(256), 0, s, reinterpret_cast<const uint4*>(p),
                     bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : -10;
}
#endif

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
  D.ctr = reinterpret_cast<int*>(take(sizeof(int) * (size_t)kLine * (1 + (size_t)kCtrLines * kDecMaxM)));
  // flag copies: kRep blocks of kDecMaxM lines, 4 KB + 256 B apart at least
  D.rstride = (int)((((size_t)kDecMaxM * kLine * sizeof(int) + 4095) / 4096 * 4096 + 256) / sizeof(int));
  D.ready = reinterpret_cast<int*>(take(sizeof(int) * (size_t)kRep * D.rstride));
  D.epoch = reinterpret_cast<int*>(take(sizeof(int) * 4));
  D.hext = D.epoch ? D.epoch + 1 : nullptr;
  D.hstride = kSegStride * (L.has_shared && L.Is > L.I ? (L.Is + kGRows - 1) / kGRows
                                                        : (L.I + kGRows - 1) / kGRows);
  D.hreg = (size_t)kHCopies * kFusedMaxM * S * D.hstride;
  D.hb = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 2 * D.hreg));
  D.sgb = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 2 * kFusedMaxM));
  // logit copies kFusedMaxM x E each, 4 KB + 256 B apart at least (on other channels)
  D.lstride = (int)((((size_t)kFusedMaxM * L.E * sizeof(uint64_t) + 4095) / 4096 * 4096 + 256) /
                    sizeof(uint64_t));
  D.logits = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * 2 * kLogitCopies * (size_t)D.lstride));
  // selection copies kFusedMaxM x kMaxTopK pairs each (every pair on a line
  // of its own: each slot's is written by another unit), 4 KB + 256 B apart
  // at least
  D.sstride = (int)((((size_t)kFusedMaxM * kMaxTopK * kSelLine * sizeof(uint64_t) + 4095) / 4096 * 4096 + 256) /
                    sizeof(uint64_t));
  D.selw = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * 2 * kSelCopies * (size_t)D.sstride));
  D.dctr = reinterpret_cast<int*>(take(sizeof(int) * (size_t)kLine * (1 + kFan)));
  D.route_ctr = reinterpret_cast<int*>(take(route_ctr_bytes()));
  D.bcounts = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)L.E));
  D.bytes = off;
  return D;
}

// output rows per D unit: 2 kDRows for 2- and 4-bit layers whose units at
// kDRows rows would outnumber the blocks resident at once (two 8-wave units
// per CU: those kernels take more than 80 VGPRs), so that most D units are
// resident from the start and prefetch their rows while the gate/up units
// stream; kDRows otherwise (and for 8-bit layers, whose 80-VGPR form keeps
// three units per CU)
static int d_rows(const DecodeLayer& L, int M, int K, bool routed) {
  if (L.gate.bits == 8 || L.H % (2 * kDRows) || d_sb_words_dev(L, K, 2 * kDRows) > kThreads) return kDRows;
  // (a thread's rows double with the unit's; kept where a D row spans more
  // than 4 chunks per lane, whose threads already hold kDRows rows each)
  const int cpc = 128 / L.gate.bits;
  if (K * (L.I / cpc) + (L.has_shared ? L.Is / cpc : 0) > 4 * kWave) return kDRows;
  const int ng = M * (K * ((L.I + kGRows - 1) / kGRows) + (L.has_shared ? (L.Is + kGRows - 1) / kGRows : 0));
  const int nr = routed ? (L.E + kRRows - 1) / kRRows : 0;
  const int nd = M * (L.H / kDRows);
  return nr + ng + nd > 2 * kCUs ? 2 * kDRows : kDRows;
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
  P.dr = d_rows(L, M, K, routed);
  P.nc = (L.H + P.dr - 1) / P.dr;
  P.d_units = M * P.nc;
  P.r_units = routed ? (L.E + kRRows - 1) / kRRows : 0;
  P.r_half = 0;
  if (routed) {
    // up to 32 R units on XCDs 0 and 1 (an even count; a unit past the last
    // row publishes nothing) when the grid reaches their blocks; more are
    // spread over every XCD in block order
    const int r2 = (P.r_units + 1) & ~1;
    if (r2 <= 32 && 8 * (r2 / 2 - 1) + 1 < r2 + P.g_units + P.d_units) {
      P.r_units = r2;
      P.r_half = r2 / 2;
    }
  }
  const DecState D = dec_state(L, K, ws);
  P.ctr = D.ctr;
  P.ready = D.ready;
  P.rstride = D.rstride;
  P.epoch = D.epoch;
  P.hext = D.hext;
  P.hb = D.hb;
  P.hreg = D.hreg;
  P.hstride = D.hstride;
  P.sgb = D.sgb;
  P.logits = D.logits;
  P.lstride = D.lstride;
  P.selw = D.selw;
  P.sstride = D.sstride;
  P.dctr = D.dctr;
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

static int d_sb_words(const DecodeLayer& L, int K, int dr) { return d_sb_words_dev(L, K, dr); }

static size_t dec_lds_bytes(const DecodeLayer& L, int K, bool routed, int M) {
  // G: x (H floats) + chunk sums (<= H/16) + 4 x 16 rows x groups bf16;
  // D: h of all S slots (S x Imax floats) + their chunk sums (<= 1/16 of that)
  //    + the staged scale/bias words;
  // with routing in the launch, G also holds the token's E router keys and
  // logits while it selects, and R units the x of the M tokens
  const size_t sel = routed ? 16 * (size_t)L.E : 0;
  const size_t g = sizeof(float) * (L.H + pad4(L.H / 16)) + 2 * 4 * kGRows * (L.H / L.gate.group_size) + sel;
  const int S = K + (L.has_shared ? 1 : 0);
  const int Im = L.has_shared && L.Is > L.I ? L.Is : L.I;
  const size_t d = sizeof(float) * ((size_t)S * Im + pad4(S * Im / 16)) +
                   16 * (size_t)d_sb_words(L, K, d_rows(L, M, K, routed));
  const size_t rx = routed ? sizeof(float) * (size_t)M * L.H : 0;
  size_t m = g > d ? g : d;
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
  if (d_sb_words(L, K, 2 * kDRows) > kThreads) return false;
  return dec_lds_bytes(L, K, false, 1) <= 160 * 1024;
}

bool fused_supported(const DecodeLayer& L, const QT& router, int M, int K) {
  // the 80-register form (8-bit, rows of at most 2 chunks per lane, D rows of
  // at most 6) polls at most 4 logits per lane: E <= 256
  const bool narrow = L.gate.bits == 8 && g_cpl(L.H, 8) <= 2 && d_ch(L, K) <= 6;
  return decode_supported(L, K) && router.bits == 8 && router.rows == L.E && router.cols == L.H &&
         M >= 1 && M <= kFusedMaxM && L.E <= (narrow ? 4 * kWave : kMaxExperts) &&
         dec_lds_bytes(L, K, true, M) <= 160 * 1024;
}

template <int B, int CPL, int DCH, int DR, bool FUSED, bool NORM>
static void run_dec(const DecodeLayer& L, const DecPlan& P, const RouteIn& R, const float* x,
                    const int32_t* idx, const float* w, const float* residual, float* y,
                    hipStream_t s) {
  const size_t lds = dec_lds_bytes(L, P.K, FUSED, P.M);
  hipLaunchKernelGGL((k_moe_decode<B, CPL, DCH, DR, FUSED, NORM>), dim3(P.r_units + P.g_units + P.d_units),
                     dim3(kThreads), lds, s, L, P, R, x, idx, w, residual, y);
}

template <bool FUSED, bool NORM = false>
static int dispatch_dec(const DecodeLayer& L, const DecPlan& P, const RouteIn& R, const float* x,
                        const int32_t* idx, const float* w, const float* residual, float* y,
                        hipStream_t s) {
  const int b = L.gate.bits;
  const int cpl = g_cpl(L.H, b);
  const int dch = d_ch(L, P.K);
#define MOEQ_DEC(B_, C_, D_)                                                            \
  if (b == B_ && cpl == C_ && dch == D_) {                                             \
    if (B_ != 8 && P.dr == 2 * kDRows)                                                 \
      run_dec<B_, C_, D_, (B_ != 8 ? 2 : 1) * kDRows, FUSED, NORM>(L, P, R, x, idx, w, residual, y, s); \
    else                                                                               \
      run_dec<B_, C_, D_, kDRows, FUSED, NORM>(L, P, R, x, idx, w, residual, y, s);   \
    return 0;                                                                          \
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
