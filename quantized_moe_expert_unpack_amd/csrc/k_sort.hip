// Group (token, slot) pairs by expert on the device, stably by pair id, and
// build the per-expert tile list of the gather GEMMs.
//
// ml-explore/mlx issue #3856 (minimal repro and the mlx-lm SwitchGLU path)
// sorts the expert indices before gather_qmm; the unsort reads back only the
// original rows.  All row counts and offsets here are int32 and every tile
// records its exact row count, so ragged tails of any length are covered (the
// issue's defect came from narrowing a remaining-row count to 16 bits).
#include "common.h"
#include "launch.h"

namespace moeq {

// counts[e] = #{p : idx[p] == e}; one block per expert.
__global__ void __launch_bounds__(256) k_count(const int32_t* __restrict__ idx, int n,
                                               int32_t* __restrict__ counts) {
  __shared__ int part[256 / kWave];
  const int e = blockIdx.x;
  int c = 0;
  for (int p = threadIdx.x; p < n; p += blockDim.x) c += idx[p] == e;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int w = 0; w < (int)(blockDim.x / kWave); ++w) s += part[w];
    counts[e] = s;
  }
}

// Exclusive scans of counts and of tiles per expert; one block of 1024.
__global__ void __launch_bounds__(1024) k_scan(const int32_t* __restrict__ counts, int E, int bm,
                                               int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ tile_off,
                                               int32_t* __restrict__ n_tiles) {
  __shared__ int sc[1024];
  __shared__ int st[1024];
  const int e = threadIdx.x;
  const int c = e < E ? counts[e] : 0;
  sc[e] = c;
  st[e] = (c + bm - 1) / bm;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // Hillis-Steele inclusive scan
    const int a = e >= o ? sc[e - o] : 0;
    const int b = e >= o ? st[e - o] : 0;
    __syncthreads();
    sc[e] += a;
    st[e] += b;
    __syncthreads();
  }
  if (e < E) {
    offsets[e + 1] = sc[e];
    tile_off[e + 1] = st[e];
  }
  if (e == 0) {
    offsets[0] = 0;
    tile_off[0] = 0;
    n_tiles[0] = st[E - 1];
  }
}

// Stable scatter: block e walks the pairs in order and appends those routed to
// e; then writes e's tiles {e, first sorted row, rows, 0}.
__global__ void __launch_bounds__(256) k_scatter(const int32_t* __restrict__ idx, int n, int bm,
                                                 const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ tile_off,
                                                 int32_t* __restrict__ sorted,
                                                 int4* __restrict__ tiles) {
  __shared__ int wave_tot[256 / kWave];
  const int e = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  const int base0 = offsets[e];
  int run = 0;
  for (int p0 = 0; p0 < n; p0 += blockDim.x) {
    const int p = p0 + threadIdx.x;
    const bool hit = p < n && idx[p] == e;
    const unsigned long long m = __ballot(hit);
    const int pre = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wave_tot[wid] = __popcll(m);
    __syncthreads();
    int before = 0, tot = 0;
    for (int w = 0; w < nw; ++w) {
      before += w < wid ? wave_tot[w] : 0;
      tot += wave_tot[w];
    }
    if (hit) sorted[base0 + run + before + pre] = p;
    run += tot;
    __syncthreads();
  }
  const int cnt = offsets[e + 1] - base0;
  const int t0 = tile_off[e];
  for (int j = threadIdx.x; j * bm < cnt; j += blockDim.x) {
    const int r0 = j * bm;
    tiles[t0 + j] = make_int4(e, base0 + r0, min(bm, cnt - r0), 0);
  }
}

int launch_sort_pairs(const int32_t* idx, int n, int E, const GatherWs& ws, hipStream_t s) {
  hipLaunchKernelGGL(k_count, dim3(E), dim3(256), 0, s, idx, n, ws.counts);
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, ws.counts, E, kGemmBM, ws.offsets,
                     ws.tile_off, ws.n_tiles);
  hipLaunchKernelGGL(k_scatter, dim3(E), dim3(256), 0, s, idx, n, kGemmBM, ws.offsets, ws.tile_off,
                     ws.sorted, ws.tiles);
  return 0;
}

}  // namespace moeq
