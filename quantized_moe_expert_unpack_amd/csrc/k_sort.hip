// Group (token, slot) pairs by expert on the device and build the per-expert
// tile list of the gather GEMMs.
//
// ml-explore/mlx issue #3856 (minimal repro and the mlx-lm SwitchGLU path)
// sorts the expert indices before gather_qmm; the unsort reads back only the
// original rows.  All row counts and offsets here are int32 and every tile
// records its exact row count, so ragged tails of any length are covered (the
// issue's defect came from narrowing a remaining-row count to 16 bits).
//
// Up to 4096 pairs, one block does it all (k_sort_small); more take three
// launches: a histogram (LDS counts per block, one global add per
// (block, expert)), a one-block scan (expert offsets, tile offsets, the tile
// list, and per-expert cursors initialised to the offsets; it also clears the
// counts for the next call) and a scatter (LDS ranks per block, one global
// cursor add per (block, expert)).  Within an expert the pair order depends on
// atomic order; a pair's GEMM output does not depend on its position in a
// tile, so results are bitwise reproducible all the same.
#include "common.h"
#include "launch.h"

namespace moeq {

constexpr int kSortThreads = 256;
constexpr int kSortChunk = 4096;   // pairs per block
constexpr int kSortMaxE = 1024;

__global__ void __launch_bounds__(kSortThreads) k_hist(const int32_t* __restrict__ idx, int n, int E,
                                                       int32_t* __restrict__ counts) {
  __shared__ int h[kSortMaxE];
  for (int e = threadIdx.x; e < E; e += kSortThreads) h[e] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * kSortChunk;
  const int p1 = min(n, p0 + kSortChunk);
  for (int p = p0 + threadIdx.x; p < p1; p += kSortThreads) {
    const int e = idx[p];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kSortThreads)
    if (h[e]) atomicAdd(&counts[e], h[e]);
}

// one block of 1024 threads; E <= 1024
__global__ void __launch_bounds__(1024) k_scan(int32_t* __restrict__ counts, int E, int bm,
                                               int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ cursor,
                                               int32_t* __restrict__ tile_off,
                                               int32_t* __restrict__ n_tiles,
                                               int4* __restrict__ tiles) {
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
    const int off = sc[e] - c;
    const int toff = st[e] - (c + bm - 1) / bm;
    offsets[e] = off;
    offsets[e + 1] = sc[e];
    cursor[e] = off;
    tile_off[e] = toff;
    tile_off[e + 1] = st[e];
    counts[e] = 0;                       // clean for the next call
    for (int j = 0; j * bm < c; ++j) tiles[toff + j] = make_int4(e, off + j * bm, min(bm, c - j * bm), 0);
  }
  if (e == 0) n_tiles[0] = st[E - 1];
}

__global__ void __launch_bounds__(kSortThreads) k_scatter(const int32_t* __restrict__ idx, int n, int E,
                                                          int32_t* __restrict__ cursor,
                                                          int32_t* __restrict__ sorted) {
  __shared__ int h[kSortMaxE];
  __shared__ int base[kSortMaxE];
  for (int e = threadIdx.x; e < E; e += kSortThreads) h[e] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * kSortChunk;
  const int p1 = min(n, p0 + kSortChunk);
  constexpr int kPer = kSortChunk / kSortThreads;
  int rank[kPer];
  int ev[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int p = p0 + threadIdx.x + j * kSortThreads;
    ev[j] = p < p1 ? idx[p] : -1;
    rank[j] = (ev[j] >= 0 && ev[j] < E) ? atomicAdd(&h[ev[j]], 1) : -1;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kSortThreads)
    if (h[e]) base[e] = atomicAdd(&cursor[e], h[e]);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (rank[j] >= 0) sorted[base[ev[j]] + rank[j]] = p0 + threadIdx.x + j * kSortThreads;
  }
}

// Up to kSortChunk pairs: the three phases in one block of 1024 threads (LDS
// counts with each pair's rank, the scan and tile list, the scatter).  The
// outputs are those of the three launches; the global counts are not used
// (they stay zero), nor the cursors.
__global__ void __launch_bounds__(1024) k_sort_small(const int32_t* __restrict__ idx, int n, int E,
                                                     int bm, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ tile_off,
                                                     int32_t* __restrict__ n_tiles,
                                                     int4* __restrict__ tiles,
                                                     int32_t* __restrict__ sorted) {
  __shared__ int sc[1024];
  __shared__ int st[1024];
  constexpr int kPer = kSortChunk / 1024;
  const int tid = threadIdx.x;
  sc[tid] = 0;
  __syncthreads();
  int rank[kPer], ev[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int p = tid + j * 1024;
    ev[j] = p < n ? idx[p] : -1;
    rank[j] = (ev[j] >= 0 && ev[j] < E) ? atomicAdd(&sc[ev[j]], 1) : -1;
  }
  __syncthreads();
  const int c = tid < E ? sc[tid] : 0;
  st[tid] = (c + bm - 1) / bm;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // Hillis-Steele inclusive scan
    const int a = tid >= o ? sc[tid - o] : 0;
    const int b = tid >= o ? st[tid - o] : 0;
    __syncthreads();
    sc[tid] += a;
    st[tid] += b;
    __syncthreads();
  }
  if (tid < E) {
    const int off = sc[tid] - c;
    const int toff = st[tid] - (c + bm - 1) / bm;
    offsets[tid] = off;
    offsets[tid + 1] = sc[tid];
    tile_off[tid] = toff;
    tile_off[tid + 1] = st[tid];
    for (int j = 0; j * bm < c; ++j) tiles[toff + j] = make_int4(tid, off + j * bm, min(bm, c - j * bm), 0);
  }
  if (tid == 0) n_tiles[0] = st[E - 1];
  // a pair's place: its expert's first row (the exclusive prefix) + its rank
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (rank[j] < 0) continue;
    const int e = ev[j];
    sorted[(e > 0 ? sc[e - 1] : 0) + rank[j]] = tid + j * 1024;
  }
}

// Indices already non-decreasing (gather_qmm with sorted indices): the rows
// stay where they are (sorted[i] = i) and expert e owns the run of rows
// [offsets[e], offsets[e+1]).  Thread i in [0, n] looks at the step from index
// i-1 to index i (an index below 0 reads as -1, one at or above E as E, and
// the two ends as -1 and E): each expert that the step passes starts its run
// at row i.  For non-decreasing indices every offset is written exactly once;
// otherwise some are written by several threads, which k_scan_runs and the
// run check of k_mark_invalid make harmless.
__global__ void __launch_bounds__(kSortThreads) k_runs(const int32_t* __restrict__ idx, int n, int E,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ sorted) {
  const int i = blockIdx.x * kSortThreads + threadIdx.x;
  if (i > n) return;
  auto clamp_e = [E](int v) { return v < 0 ? -1 : (v >= E ? E : v); };
  const int prev = i > 0 ? clamp_e(idx[i - 1]) : -1;
  const int cur = i < n ? clamp_e(idx[i]) : E;
  for (int e = prev + 1; e <= cur; ++e) offsets[e] = i;
  if (i < n) sorted[i] = i;
}

// one block of 1024 threads, E <= 1024: the run starts made non-decreasing (a
// running maximum: with non-decreasing indices they already are), then the
// tile list of k_scan from the run lengths
__global__ void __launch_bounds__(1024) k_scan_runs(int32_t* __restrict__ offsets, int E, int bm,
                                                    int32_t* __restrict__ tile_off,
                                                    int32_t* __restrict__ n_tiles,
                                                    int4* __restrict__ tiles) {
  __shared__ int so[1024];
  __shared__ int st[1024];
  __shared__ int s_end;
  const int e = threadIdx.x;
  so[e] = e < E ? offsets[e] : 0;
  if (e == 0) s_end = offsets[E];
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive running maximum
    const int a = e >= o ? so[e - o] : 0;
    __syncthreads();
    so[e] = max(so[e], a);
    __syncthreads();
  }
  const int last = max(s_end, so[E - 1]);
  const int start = so[e];
  const int c = e < E ? (e + 1 < E ? so[e + 1] : last) - start : 0;
  st[e] = (c + bm - 1) / bm;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // Hillis-Steele inclusive scan
    const int b = e >= o ? st[e - o] : 0;
    __syncthreads();
    st[e] += b;
    __syncthreads();
  }
  if (e < E) {
    const int toff = st[e] - (c + bm - 1) / bm;
    offsets[e] = start;
    tile_off[e] = toff;
    tile_off[e + 1] = st[e];
    for (int j = 0; j * bm < c; ++j) tiles[toff + j] = make_int4(e, start + j * bm, min(bm, c - j * bm), 0);
  }
  if (e == 0) {
    offsets[E] = last;
    n_tiles[0] = st[E - 1];
  }
}

int launch_runs(const int32_t* idx, int n, int E, const GatherWs& ws, hipStream_t s) {
  const int blocks = (n + 1 + kSortThreads - 1) / kSortThreads;
  hipLaunchKernelGGL(k_runs, dim3(blocks), dim3(kSortThreads), 0, s, idx, n, E, ws.offsets, ws.sorted);
  hipLaunchKernelGGL(k_scan_runs, dim3(1), dim3(1024), 0, s, ws.offsets, E, kGemmBM, ws.tile_off,
                     ws.n_tiles, ws.tiles);
  return 0;
}

int launch_sort_pairs(const int32_t* idx, int n, int E, const GatherWs& ws, hipStream_t s) {
  return launch_sort_pairs_bm(idx, n, E, ws, kGemmBM, s);
}

int launch_sort_pairs_bm(const int32_t* idx, int n, int E, const GatherWs& ws, int bm, hipStream_t s) {
  if (n <= kSortChunk) {
    hipLaunchKernelGGL(k_sort_small, dim3(1), dim3(1024), 0, s, idx, n, E, bm, ws.offsets,
                       ws.tile_off, ws.n_tiles, ws.tiles, ws.sorted);
    return 0;
  }
  const int blocks = (n + kSortChunk - 1) / kSortChunk;
  hipLaunchKernelGGL(k_hist, dim3(blocks), dim3(kSortThreads), 0, s, idx, n, E, ws.counts);
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, ws.counts, E, bm, ws.offsets,
                     ws.cursor, ws.tile_off, ws.n_tiles, ws.tiles);
  hipLaunchKernelGGL(k_scatter, dim3(blocks), dim3(kSortThreads), 0, s, idx, n, E, ws.cursor,
                     ws.sorted);
  return 0;
}

}  // namespace moeq
