// Internal interface between the C-ABI front end (abi.cpp) and the kernel
// translation units.  Launchers assume validated arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace moeq {

constexpr int kMaxLdsBytes = 160 * 1024;   // LDS of one gfx950 CU

// Allow a kernel all the LDS its static shared arrays leave free as dynamic
// shared memory, once per device: the limit is an attribute of the kernel, so
// setting it on every launch would only add host work.  `done` is the call
// site's own static bit set.
// `need` is the launch's own dynamic LDS: if the runtime refuses the larger
// limit, its error is taken back and the launch's size is set instead (then
// on every launch, as the limit does not cover other sizes).
inline void allow_full_lds(const void* kernel, int need, std::atomic<uint64_t>& done) {
  int dev = 0;
  (void)hipGetDevice(&dev);
  const uint64_t bit = 1ull << (dev & 63);
  if (done.load(std::memory_order_acquire) & bit) return;
  hipFuncAttributes a{};
  if (hipFuncGetAttributes(&a, kernel) == hipSuccess &&
      hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                          kMaxLdsBytes - (int)a.sharedSizeBytes) == hipSuccess) {
    done.fetch_or(bit, std::memory_order_acq_rel);
    return;
  }
  (void)hipGetLastError();   // the refusal above, not a launch failure
  (void)hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, need);
}
#define MOEQ_ALLOW_FULL_LDS(kernel, need)                \
  do {                                                   \
    static std::atomic<uint64_t> moeq_lds_once_{0};      \
    ::moeq::allow_full_lds((const void*)(kernel), (int)(need), moeq_lds_once_); \
  } while (0)

// A validated quantized tensor (see moeq_qtensor in include/moeq.h).
struct QT {
  const uint32_t* q;
  const uint16_t* scales;
  const uint16_t* biases;
  int batch, rows, cols, bits, group_size;
  int mode;   // 0 affine; 1 mxfp4 (E2M1 codes, uint8 E8M0 scales in `scales`, no biases)
};

// Decode (fp32 activations) layer description.
struct DecodeLayer {
  QT gate, up, down;   // [E][I][H], [E][I][H], [E][H][I]
  int has_shared;
  QT sh_gate, sh_up, sh_down, sh_eg;  // [1][Is][H] x2, [1][H][Is], [1][1][H]
  int E, H, I, Is;
};

// Decode-family workspaces (moe_expert_forward, moe_forward) start with this
// state block.  Its layout depends on the layer's shape and K only, never on
// M, so one workspace serves calls of any M up to the size it was made for:
// every word here holds zero between calls (the kernels clear what they set),
// except the one-launch form's launch counter and its two extent words.
constexpr int kDecMaxM = 16;   // tokens per per-token decode launch (more go in chunks)
constexpr int kFusedMaxM = 4;  // tokens of the one-launch (routing inside) form
struct DecState {
  int* ctr;          // error word, then per-token arrival counters (kDecMaxM tokens)
  int* ready;        // ready-flag copies
  int rstride;       // ints between copies
  int* epoch;        // one-launch counter; its parity picks the h buffer
  int* hext;         // [2] 16-byte words of each h buffer the last launch using it wrote
  uint32_t* hb;      // [2][hreg] complemented-bit h buffers of the one-launch form
  size_t hreg;       // words per h buffer
  int hstride;       // words per (copy, pair) row of an h buffer (segments on 128-byte lines)
  uint32_t* sgb;     // [2][kFusedMaxM] shared-gate logits, the same way
  uint64_t* logits;  // [2 parities][copies][lstride] complemented fp64 logits [kFusedMaxM][E], 0 = not written
  int lstride;       // u64 words per logit copy
  uint64_t* selw;    // [2 parities][copies][sstride]: [kFusedMaxM][kMaxTopK] complemented
                     // (expert << 32 | fp32 weight bits) of every slot, 0 = not written,
                     // each pair at the start of a 128-byte line of its own
  int sstride;
  int* dctr;         // arrival counter lines of the one-launch form's D units (the launch's last one)
  int* route_ctr;    // counters of a separate routing launch
  int32_t* bcounts;  // [E] per-expert pair counts of the batched form
  size_t bytes;      // size of the block (256-byte multiple)
};
DecState dec_state(const DecodeLayer& L, int K, void* ws);

// Decode plan: unit counts, the state block above and the launch's data.
struct DecPlan {
  int M, K, S, P, Imax;
  int ng_routed, ng_shared, g_units, nc, d_units;
  int dr;          // output rows per D unit
  int r_units;     // router units in front of the expert units (routing in the launch), else 0
  int r_half;      // R units per XCD on XCDs 0 and 1 (block placement), 0: R units first in order
  int* ctr;        // 128-byte lines: error word, then per token G and D arrival counters
  int* ready;      // ready flags: copies [kRep] of token lines, rstride ints apart
  int rstride;
  float* h;        // [copies][P][Imax] (pair p = token * S + slot)
  float* sg;       // [M]
  uint64_t* logits;  // [2 parities][copies][lstride]: router logits [kFusedMaxM][E] as complemented
                     // fp64 bits, 0 = not written
  int lstride;
  uint64_t* selw;    // [2 parities][copies][sstride]: every slot's (expert << 32 | fp32 weight
                     // bits), complemented, 0 = not written; [kFusedMaxM][kMaxTopK] per copy,
                     // each pair at the start of a 128-byte line of its own
  int sstride;
  int* dctr;         // arrival counter lines of the D units (the launch's last one moves epoch on)
  int* epoch;        // launch counter (routing in the launch): its parity picks the h buffer
  int* hext;         // [2] extent (16-byte words) of each h buffer's last use
  uint32_t* hb;      // [2][hreg]: [copies][P][hstride] h as complemented fp32 bits, 0 = not written
  size_t hreg;
  int hstride;       // segments of kGRows values, each at the front of a 128-byte line
  uint32_t* sgb;     // [2][kFusedMaxM] shared-gate logits, the same way
  const float* norm_w;  // RMSNorm weight [H] of a launch that normalizes x first, else null
  float norm_eps;
};

// Router of a decode launch that routes in the same launch.
struct RouteIn {
  QT W;            // [E][H], 8-bit
  int renorm;
  int32_t* idx_out;  // [M][K] (caller's)
  float* w_out;      // [M][K] (caller's)
};

// Workspace carve-up for the gather (prefill) path; every pointer is
// 256-byte aligned inside the caller's workspace.
struct GatherWs {
  int32_t* counts;     // [E]    zero between calls
  int32_t* offsets;    // [E+1]  sorted row offset per expert
  int32_t* cursor;     // [E]    scatter cursors
  int32_t* tile_off;   // [E+1]  first tile per expert
  int32_t* n_tiles;    // [1]
  int4* tiles;         // [max_tiles] {expert, row0, rows, 0}
  int32_t* sorted;     // [n] pair id at each sorted position
  uint16_t* h;         // [n][I] bf16 (moe_gather_qmm only)
  uint16_t* ypair;     // [n][H] bf16 (moe_gather_qmm only)
  int max_tiles;
};

constexpr int kGemmBM = 256;  // rows per gather-GEMM tile

// Batched decode (many fp32 tokens; k_batch.hip): pairs grouped by expert in
// tiles of at most kBTile pairs; a unit applies its rows to kBTok tokens.
constexpr int kBTok = 2;
constexpr int kBTile = kBTok;
constexpr int kBatchMinM = 16;   // from this many tokens moe_expert_forward batches by expert
struct BatchWs {
  GatherWs sort;         // pair sort by expert (tiles of kBTile rows)
  int max_tiles;
  const int32_t* n_tiles;
  const int4* tiles;
  const int32_t* sorted;
  float* h;              // [n][I]
  float* hsh;            // [M][Is]
  float* sg;             // [M]
  float* ypair;          // [n][H]
  float* ysh;            // [M][H]
};

int launch_qdequant(const QT& W, uint8_t* codes, float* deq, hipStream_t s);
int launch_qmatvec(const QT& W, const float* x, int M, float* y, hipStream_t s);
// RMSNorm per row: h = x / sqrt(mean(x^2) + eps) * g, rows of H (H % 4 == 0)
int launch_rmsnorm(const float* x, int M, int H, const float* g, float eps, float* h, hipStream_t s);
// 2-bit requantization of a 4- or 8-bit tensor (group size 64 or 128)
int launch_requant_2bit(const QT& W, uint32_t* q2, uint16_t* s2, uint16_t* b2, hipStream_t s);
// routing: router projection (fp64) + softmax/top-K.  The standalone
// workspace is [counters (zero between calls)][fp64 logits [M][E]].
size_t route_ctr_bytes();
size_t route_ws_bytes(int M, int E);
int launch_route(const QT* router, const float* x_or_logits, int M, int E, int K, int renorm,
                 int32_t* idx, float* w, float* logits32, void* ws, hipStream_t s);
int launch_route_parts(const QT* router, const float* x_or_logits, int M, int E, int K, int renorm,
                       int32_t* idx, float* w, float* logits32, double* l64, int* ctr,
                       hipStream_t s);

// decode expert forward (one launch, M <= kDecMaxM); the workspace is the
// state block followed by the launch's data
int launch_decode_forward(const DecodeLayer& L, const float* x, const int32_t* idx, const float* w,
                          int M, int K, const float* residual, float* y, void* ws, hipStream_t s);
size_t decode_ws_bytes(const DecodeLayer& L, int M, int K, bool routed_in_launch = false);
bool decode_supported(const DecodeLayer& L, int K);
// router + experts in one launch (8-bit router, M <= kFusedMaxM)
bool fused_supported(const DecodeLayer& L, const QT& router, int M, int K);
int launch_moe_forward(const DecodeLayer& L, const RouteIn& R, const float* x, int M, int K,
                       const float* residual, float* y, void* ws, hipStream_t s);
int launch_moe_forward_norm(const DecodeLayer& L, const RouteIn& R, const float* x, int M, int K,
                            const float* norm_w, float eps, float* y, void* ws, hipStream_t s);

// the error word of a decode-family workspace: out[0] = 0 or `timeout_status`,
// out[1] = its bits; then the word is cleared (one thread, stream-ordered)
int launch_ws_status(void* ws, int32_t* out, int timeout_status, hipStream_t s);

// batched decode
bool batch_supported(const DecodeLayer& L);
int launch_batch_forward(const DecodeLayer& L, const float* x, const int32_t* idx, const float* w,
                         int M, int K, const float* residual, float* y, const BatchWs& B,
                         hipStream_t s);

// gather path
int launch_sort_pairs(const int32_t* idx, int n, int E, const GatherWs& ws, hipStream_t s);
int launch_sort_pairs_bm(const int32_t* idx, int n, int E, const GatherWs& ws, int bm, hipStream_t s);
int launch_gemm_gate_up(const QT& gate, const QT& up, const uint16_t* x, int K, const GatherWs& ws,
                        int n, hipStream_t s);
int launch_gemm_down(const QT& down, const float* w, const GatherWs& ws, int n, hipStream_t s);
int launch_gemm_plain(const QT& W, const uint16_t* x, float* out, const GatherWs& ws, int n,
                      hipStream_t s);
// indices already non-decreasing: rows used in place, each expert's run of
// rows as its tiles (no sort)
int launch_runs(const int32_t* idx, int n, int E, const GatherWs& ws, hipStream_t s);
// rows whose expert index is outside [0, E) become NaN (gather_qmm output);
// with runs (the offsets of launch_runs) also rows outside their expert's run
int launch_mark_invalid_rows(const int32_t* idx, int n, int E, int N, const int32_t* runs, float* out,
                             hipStream_t s);
int launch_combine(const uint16_t* ypair, const int32_t* idx, int M, int K, int H, int E, float* y,
                   hipStream_t s);

}  // namespace moeq
