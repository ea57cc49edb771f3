// C-ABI front end of libmoeq: argument validation (before any launch),
// workspace carve-up and dispatch to the HIP kernels.  See include/moeq.h for
// the contract of every entry point.
#include "moeq.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>
#include <mutex>
#include <vector>

#include "launch.h"
#include "stream.h"

namespace moeq {
// bf16 -> fp32 widening of n values (k_matvec.hip)
int launch_bf16_widen(const uint16_t* x, float* y, int64_t n, hipStream_t s);
}  // namespace moeq

using moeq::QT;

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxE = 1024;
constexpr int kMaxK = 16;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool fits_i32(int64_t v) { return v >= 0 && v <= INT32_MAX; }

// Validate one quantized tensor; expected dims < 0 are not checked.
int check_qt(const moeq_qtensor* t, int batch, int rows, int cols) {
  if (!t) return MOEQ_ERR_NULL_PTR;
  if (t->mode != MOEQ_MODE_AFFINE && t->mode != MOEQ_MODE_MXFP4) return MOEQ_ERR_UNSUPPORTED;
  const bool mx = t->mode == MOEQ_MODE_MXFP4;
  if (!t->q || !t->scales || (!mx && !t->biases)) return MOEQ_ERR_NULL_PTR;
  if (mx) {
    if (t->bits != 4) return MOEQ_ERR_BAD_BITS;
    if (t->group_size != 32) return MOEQ_ERR_BAD_GROUP;
  }
  if (t->bits != 2 && t->bits != 4 && t->bits != 8) return MOEQ_ERR_BAD_BITS;
  // 32, 64 or 128 elements per group; at 2 bits 64 or 128 (a 16-byte chunk
  // of 2-bit codes is 64 elements and must lie in one group)
  if (t->group_size != 32 && t->group_size != 64 && t->group_size != 128) return MOEQ_ERR_BAD_GROUP;
  if (t->bits == 2 && t->group_size == 32) return MOEQ_ERR_BAD_GROUP;
  if (t->batch <= 0 || t->rows <= 0 || t->cols <= 0) return MOEQ_ERR_SHAPE;
  if (t->cols % t->group_size) return MOEQ_ERR_K_TAIL;
  if (batch >= 0 && t->batch != batch) return MOEQ_ERR_SHAPE;
  if (rows >= 0 && t->rows != rows) return MOEQ_ERR_SHAPE;
  if (cols >= 0 && t->cols != cols) return MOEQ_ERR_SHAPE;
  if (!fits_i32((int64_t)t->batch * t->rows) ||
      !fits_i32((int64_t)t->batch * t->rows * (t->cols / (32 / t->bits))) ||
      !fits_i32((int64_t)t->batch * t->rows * t->cols / 4))
    return MOEQ_ERR_OVERFLOW;
  if (!aligned16(t->q) || !aligned16(t->scales) || (!mx && !aligned16(t->biases))) return MOEQ_ERR_ALIGN;
  return MOEQ_OK;
}

bool is_mx(const moeq_qtensor& t) { return t.mode == MOEQ_MODE_MXFP4; }

QT to_qt(const moeq_qtensor& t) {
  return QT{t.q, t.scales, is_mx(t) ? nullptr : t.biases, t.batch, t.rows, t.cols, t.bits,
            t.group_size, t.mode};
}

int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOEQ_OK : MOEQ_ERR_LAUNCH;
}

// ---- layer validation -----------------------------------------------------
struct LayerDims {
  int E, H, I, Is;
};

int check_experts(const moeq_moe* L, LayerDims* d) {
  if (!L) return MOEQ_ERR_NULL_PTR;
  const moeq_qtensor& g = L->gate;
  int st = check_qt(&g, -1, -1, -1);
  if (st) return st;
  d->E = g.batch;
  d->I = g.rows;
  d->H = g.cols;
  if (d->E > kMaxE) return MOEQ_ERR_SHAPE;
  if ((st = check_qt(&L->up, d->E, d->I, d->H))) return st;
  if ((st = check_qt(&L->down, d->E, d->H, d->I))) return st;
  if (L->up.bits != g.bits || L->down.bits != g.bits) return MOEQ_ERR_UNSUPPORTED;
  if (L->up.mode != g.mode || L->down.mode != g.mode) return MOEQ_ERR_UNSUPPORTED;
  // one group size for every expert matrix (the router and the shared
  // expert's gate row may differ)
  if (L->up.group_size != g.group_size || L->down.group_size != g.group_size)
    return MOEQ_ERR_UNSUPPORTED;
  d->Is = 0;
  if (L->has_shared) {
    if ((st = check_qt(&L->sh_gate, 1, -1, d->H))) return st;
    d->Is = L->sh_gate.rows;
    if ((st = check_qt(&L->sh_up, 1, d->Is, d->H))) return st;
    if ((st = check_qt(&L->sh_down, 1, d->H, d->Is))) return st;
    if ((st = check_qt(&L->sh_expert_gate, 1, 1, d->H))) return st;
    if (L->sh_up.bits != L->sh_gate.bits || L->sh_down.bits != L->sh_gate.bits)
      return MOEQ_ERR_UNSUPPORTED;
    if (is_mx(L->sh_gate) || is_mx(L->sh_up) || is_mx(L->sh_down) || is_mx(L->sh_expert_gate))
      return MOEQ_ERR_UNSUPPORTED;                    // the shared expert is affine
    if (L->sh_gate.group_size != g.group_size || L->sh_up.group_size != g.group_size ||
        L->sh_down.group_size != g.group_size)
      return MOEQ_ERR_UNSUPPORTED;
  }
  return MOEQ_OK;
}

// ---- workspace layouts ----------------------------------------------------
moeq::DecodeLayer to_decode_layer(const moeq_moe* L, const LayerDims& d) {
  moeq::DecodeLayer dl;
  dl.gate = to_qt(L->gate);
  dl.up = to_qt(L->up);
  dl.down = to_qt(L->down);
  dl.has_shared = L->has_shared ? 1 : 0;
  if (dl.has_shared) {
    dl.sh_gate = to_qt(L->sh_gate);
    dl.sh_up = to_qt(L->sh_up);
    dl.sh_down = to_qt(L->sh_down);
    dl.sh_eg = to_qt(L->sh_expert_gate);
  } else {
    dl.sh_gate = dl.sh_up = dl.sh_down = dl.sh_eg = dl.gate;
  }
  dl.E = d.E;
  dl.H = d.H;
  dl.I = d.I;
  dl.Is = d.Is;
  return dl;
}

int max_tiles_for(int n, int E) { return (n + moeq::kGemmBM - 1) / moeq::kGemmBM + E; }

// carve the gather workspace; with base == nullptr only the size is computed
size_t gather_ws(char* base, int E, int n, int I, int H, bool full, moeq::GatherWs* ws) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  moeq::GatherWs w{};
  w.max_tiles = max_tiles_for(n, E);
  w.counts = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * E));
  w.offsets = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (E + 1)));
  w.cursor = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * E));
  w.tile_off = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (E + 1)));
  w.n_tiles = reinterpret_cast<int32_t*>(take(sizeof(int32_t)));
  w.tiles = reinterpret_cast<int4*>(take(sizeof(int4) * (size_t)w.max_tiles));
  w.sorted = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)n));
  if (full) {
    w.h = reinterpret_cast<uint16_t*>(take(sizeof(uint16_t) * (size_t)n * I));
    w.ypair = reinterpret_cast<uint16_t*>(take(sizeof(uint16_t) * (size_t)n * H));
  }
  if (ws) *ws = w;
  return off;
}

// carve the batched-decode workspace (pairs sorted by expert in tiles of
// kBTile rows); with base == nullptr only the size is computed.  skip bytes
// after the state block are left alone (moe_gather_qmm keeps its own
// counters there)
size_t batch_ws(char* base, const moeq::DecodeLayer& dl, int M, int K, moeq::BatchWs* out,
                size_t skip = 0) {
  // the decode state block first (its per-expert counts serve the sort)
  const moeq::DecState st = moeq::dec_state(dl, K, base);
  size_t off = st.bytes + skip;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  const int n = M * K, E = dl.E;
  moeq::GatherWs w{};
  // each expert's rows make ceil(rows / kBTile) tiles, each tile has a row
  const int mt = (n + moeq::kBTile - 1) / moeq::kBTile + E;
  w.max_tiles = mt < n ? mt : n;
  w.counts = st.bcounts;
  w.offsets = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (E + 1)));
  w.cursor = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * E));
  w.tile_off = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (E + 1)));
  w.n_tiles = reinterpret_cast<int32_t*>(take(sizeof(int32_t)));
  w.tiles = reinterpret_cast<int4*>(take(sizeof(int4) * (size_t)w.max_tiles));
  w.sorted = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)n));
  moeq::BatchWs b{};
  b.sort = w;
  b.max_tiles = w.max_tiles;
  b.n_tiles = w.n_tiles;
  b.tiles = w.tiles;
  b.sorted = w.sorted;
  b.h = reinterpret_cast<float*>(take(sizeof(float) * (size_t)n * dl.I));
  b.hsh = reinterpret_cast<float*>(take(sizeof(float) * (size_t)M * (dl.Is > 0 ? dl.Is : 1)));
  b.sg = reinterpret_cast<float*>(take(sizeof(float) * (size_t)M));
  b.ypair = reinterpret_cast<float*>(take(sizeof(float) * (size_t)n * dl.H));
  b.ysh = reinterpret_cast<float*>(take(sizeof(float) * (size_t)M * dl.H));
  if (out) *out = b;
  return off;
}

bool use_batch(const moeq::DecodeLayer& dl, int M) {
  return M >= moeq::kBatchMinM && moeq::batch_supported(dl);
}

// moe_expert_forward's workspace: per-token decode launches (at most
// kDecMaxM tokens each) or batched by expert; both start with the decode
// state block
size_t expert_ws_bytes(const moeq::DecodeLayer& dl, int M, int K) {
  return use_batch(dl, M) ? batch_ws(nullptr, dl, M, K, nullptr)
                          : moeq::decode_ws_bytes(dl, M < moeq::kDecMaxM ? M : moeq::kDecMaxM, K);
}

// the expert part for given indices: batched by expert for many tokens, else
// per-token launches of at most kDecMaxM tokens, in order on the stream
int run_expert_forward(const moeq::DecodeLayer& dl, const float* x, const int32_t* idx,
                       const float* w, int M, int K, const float* residual, float* y, void* ws,
                       hipStream_t s) {
  if (use_batch(dl, M)) {
    moeq::BatchWs b;
    batch_ws(reinterpret_cast<char*>(ws), dl, M, K, &b);
    return moeq::launch_batch_forward(dl, x, idx, w, M, K, residual, y, b, s);
  }
  for (int t0 = 0; t0 < M; t0 += moeq::kDecMaxM) {
    const int m = M - t0 < moeq::kDecMaxM ? M - t0 : moeq::kDecMaxM;
    const size_t xo = (size_t)t0 * dl.H, ko = (size_t)t0 * K;
    const int st = moeq::launch_decode_forward(dl, x + xo, idx + ko, w + ko, m, K,
                                               residual ? residual + xo : nullptr, y + xo, ws, s);
    if (st) return st;
  }
  return 0;
}

// moe_forward: one launch (routing in the launch), or a routing launch and
// moe_expert_forward: [decode state block | expert data | fp64 logits], the
// routing counters inside the state block; room for either
size_t forward_ws_bytes(const moeq::DecodeLayer& dl, int E, int M, int K) {
  const size_t one = moeq::decode_ws_bytes(dl, M < moeq::kFusedMaxM ? M : moeq::kFusedMaxM, K, true);
  const size_t two = align_up(expert_ws_bytes(dl, M, K)) + align_up(moeq::route_ws_bytes(M, E));
  return one > two ? one : two;
}

// moe_forward_norm: moe_forward's workspace, then the normalized rows [M][H]
// (used when the step does not run as one launch)
size_t forward_norm_ws_bytes(const moeq::DecodeLayer& dl, int E, int M, int K) {
  return align_up(forward_ws_bytes(dl, E, M, K)) + align_up(sizeof(float) * (size_t)M * dl.H);
}

bool bad_eps(float eps) { return !(eps >= 0.0f) || eps > 3.0e38f; }

// moe_forward's argument checks: 1 when the call has work, 0 (MOEQ_OK) for
// M == 0, else the error status
int check_forward(const moeq_moe* L, const float* x, int32_t M, int32_t K, const float* residual,
                  const float* y, const int32_t* topk_idx, const float* topk_w, moeq::DecodeLayer* dl,
                  int32_t* E) {
  LayerDims d;
  int st = check_experts(L, &d);
  if (st) return st;
  if (is_mx(L->gate)) return MOEQ_ERR_UNSUPPORTED;   // mxfp4 experts: gather paths only
  if ((st = check_qt(&L->router, 1, d.E, d.H))) return st;
  if (is_mx(L->router)) return MOEQ_ERR_UNSUPPORTED;
  if (M < 0 || K < 1 || K > kMaxK || K > d.E) return MOEQ_ERR_SHAPE;
  if (M == 0) return MOEQ_OK;
  if (!x || !y || !topk_idx || !topk_w) return MOEQ_ERR_NULL_PTR;
  if (!fits_i32((int64_t)M * d.H) || !fits_i32((int64_t)M * d.E) ||
      !fits_i32((int64_t)M * K * d.I + (int64_t)M * d.Is + M))
    return MOEQ_ERR_OVERFLOW;
  if (!aligned16(x) || !aligned16(y) || !aligned16(topk_idx) || !aligned16(topk_w) ||
      (residual && !aligned16(residual)))
    return MOEQ_ERR_ALIGN;
  *dl = to_decode_layer(L, d);
  if (!moeq::decode_supported(*dl, K)) return MOEQ_ERR_UNSUPPORTED;
  *E = d.E;
  return 1;
}

// moe_forward after validation, on a workspace of forward_ws_bytes
int forward_body(const moeq_moe* L, const moeq::DecodeLayer& dl, int32_t E, const float* x, int32_t M,
                 int32_t K, int32_t renorm, const float* residual, float* y, int32_t* topk_idx,
                 float* topk_w, void* ws, hipStream_t s) {
  int st;
  const QT router = to_qt(L->router);
  if (moeq::fused_supported(dl, router, M, K)) {
    const moeq::RouteIn R{router, renorm, topk_idx, topk_w};
    st = moeq::launch_moe_forward(dl, R, x, M, K, residual, y, ws, s);
  } else {
    char* base = reinterpret_cast<char*>(ws);
    const moeq::DecState ds = moeq::dec_state(dl, K, base);
    double* l64 = reinterpret_cast<double*>(base + align_up(expert_ws_bytes(dl, M, K)));
    moeq::launch_route_parts(&router, x, M, E, K, renorm, topk_idx, topk_w, nullptr, l64,
                             ds.route_ctr, s);
    st = run_expert_forward(dl, x, topk_idx, topk_w, M, K, residual, y, base, s);
  }
  if (st) return MOEQ_ERR_UNSUPPORTED;
  return launch_status();
}

}  // namespace

// ---- the allocation-free moe_forward: its workspace is a static array ------
// One array per device, held until the process ends.  Host code never uses
// the array's name as an address: each device's address comes from
// hipGetSymbolAddress (taken once per device, with that device current).
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
constexpr int kClearBlocks = 512;

// What fixes the layout of the decode state block at the array's front: the
// layer's shape, its shared expert and K (plus the bit widths and group size,
// for good measure).  A call with another layout clears the array first.
struct ScratchKey {
  int E, H, I, Is, has_shared, K, bits, group_size, router_bits;
  bool operator==(const ScratchKey& o) const {
    return E == o.E && H == o.H && I == o.I && Is == o.Is && has_shared == o.has_shared && K == o.K &&
           bits == o.bits && group_size == o.group_size && router_bits == o.router_bits;
  }
};

struct ScratchDev {
  char* ptr;        // the device's address of `scratch` (null until first use)
  bool keyed;       // a layout has been set up
  ScratchKey key;   // the layout of the last call
  size_t used;      // bytes the calls since the last clear may have touched
};

std::mutex g_scratch_mu;
ScratchDev g_scratch[kMaxDevices];

__global__ void k_scratch_zero(uint4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// clear the array when the status just written reports a timeout
__global__ void k_scratch_clear_if(const int32_t* __restrict__ status, uint4* __restrict__ p, size_t n16) {
  if (status[1] == 0) return;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

size_t scratch_used_16(const char* ws) {
  std::lock_guard<std::mutex> g(g_scratch_mu);
  for (auto& d : g_scratch)
    if (d.ptr == ws) return d.used / 16;
  return 0;
}

// The current device's scratch address for a call needing `need` bytes;
// clears (on `s`, by a fill kernel) what the previous layout used when this
// call's layout differs, and on the device's first call the whole array.
int scratch_for_call(const moeq::DecodeLayer& dl, const moeq_qtensor& router, int K, size_t need,
                     hipStream_t s, char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOEQ_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return MOEQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  ScratchDev& d = g_scratch[dev];
  if (!d.ptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOEQ_ERR_LAUNCH;
    d.ptr = static_cast<char*>(p);
    d.used = kScratchBytes;        // not known to be clear: the first call clears it all
  }
  const ScratchKey key{dl.E, dl.H, dl.I, dl.Is, dl.has_shared, K, dl.gate.bits, dl.gate.group_size,
                       router.bits};
  if (!d.keyed || !(d.key == key)) {
    const size_t n = std::max(d.used, need);
    hipLaunchKernelGGL(k_scratch_zero, dim3(kClearBlocks), dim3(256), 0, s,
                       reinterpret_cast<uint4*>(d.ptr), (n + 15) / 16);
    d.key = key;
    d.keyed = true;
    d.used = need;
  } else {
    d.used = std::max(d.used, need);
  }
  *out = d.ptr;
  return MOEQ_OK;
}

}  // namespace

extern "C" {

const char* moeq_status_string(int status) {
  switch (status) {
    case MOEQ_OK: return "ok";
    case MOEQ_ERR_NULL_PTR: return "a required pointer is NULL";
    case MOEQ_ERR_BAD_BITS: return "bits must be 2, 4 or 8";
    case MOEQ_ERR_BAD_GROUP: return "group_size must be 32, 64 or 128 (64 or 128 at 2 bits)";
    case MOEQ_ERR_K_TAIL: return "cols must be a multiple of group_size";
    case MOEQ_ERR_SHAPE: return "inconsistent shapes";
    case MOEQ_ERR_OVERFLOW: return "a size or index does not fit int32";
    case MOEQ_ERR_ALIGN: return "device pointers must be 16-byte aligned";
    case MOEQ_ERR_WORKSPACE: return "workspace missing or too small";
    case MOEQ_ERR_UNSUPPORTED: return "unsupported combination";
    case MOEQ_ERR_LAUNCH: return "kernel launch failed";
    case MOEQ_ERR_HOST_MEMORY: return "host memory is not pinned and mapped for the device";
    case MOEQ_ERR_TIMEOUT: return "a bounded wait inside a decode launch gave up (outputs wrong)";
    default: return "unknown status";
  }
}

// ---- the prefill gather with few rows per expert --------------------------
// With at most kLightPairs (token, slot) pairs per expert on average a 256-row
// MFMA tile holds a handful of rows, and the gather GEMM's cost is staging
// and dequantizing each touched expert's weights per tile; the batched decode
// kernels stream each touched expert once per tile of two pairs instead
// (measured on the 30B-A3B shapes: 2.3 pairs per expert 97 against 176 us,
// 4.9 pairs 252 against 291 us, 16 pairs 748 against 301 us).  The bf16
// activations are widened exactly to fp32 for them.
constexpr int kLightPairs = 4;

bool light_layer(const moeq_moe* L, const moeq::DecodeLayer& dl) {
  return !is_mx(L->gate) && !L->has_shared && moeq::batch_supported(dl);
}
// the largest M that takes the light form
int light_max_m(const moeq::DecodeLayer& dl, int K) { return kLightPairs * dl.E / K; }

bool light_gather(const moeq_moe* L, const moeq::DecodeLayer& dl, int M, int K) {
  return M <= light_max_m(dl, K) && light_layer(L, dl);
}

// moe_gather_qmm's workspace: the decode state block first (the light form's
// counters), then the gather GEMM's per-expert counts (both at offsets
// independent of M, zero between calls), then either the rest of the gather
// GEMM's data or the light form's batched data followed by the fp32
// activations
size_t gather_counts_bytes(int E) { return align_up(sizeof(int32_t) * (size_t)E); }

size_t gather_call_ws(const moeq::DecodeLayer& dl, int M, int K, bool light, size_t* x_off) {
  const size_t st = moeq::dec_state(dl, K, nullptr).bytes;
  const size_t heavy = st + gather_ws(nullptr, dl.E, M * K, dl.I, dl.H, true, nullptr);
  if (!light) return heavy;
  const size_t b = batch_ws(nullptr, dl, M, K, nullptr, gather_counts_bytes(dl.E));
  if (x_off) *x_off = b;
  const size_t l = b + align_up(sizeof(float) * (size_t)M * dl.H);
  return l > heavy ? l : heavy;
}

const char* moeq_version(void) { return "moeq 0.1 gfx950"; }

size_t moe_workspace_size(const moeq_moe* L, int32_t M, int32_t K, int32_t path) {
  if (!L || M < 0) return 0;
  if (path == MOEQ_PATH_ROUTE) {
    const int E = L->router.q ? L->router.rows : L->gate.batch;
    if (E <= 0) return 0;
    return moeq::route_ws_bytes(M, E) + kAlign;
  }
  if (path == MOEQ_PATH_GQMM) {
    if (check_qt(&L->gate, -1, -1, -1)) return 0;
    return gather_ws(nullptr, L->gate.batch, M, 0, 0, false, nullptr) + kAlign;
  }
  LayerDims d;
  if (check_experts(L, &d)) return 0;
  if (K < 1 || K > kMaxK || K > d.E) return 0;
  if (path == MOEQ_PATH_DECODE) return expert_ws_bytes(to_decode_layer(L, d), M, K) + kAlign;
  if (path == MOEQ_PATH_FORWARD) {
    if (!L->router.q || L->router.rows != d.E) return 0;
    return forward_ws_bytes(to_decode_layer(L, d), d.E, M, K) + kAlign;
  }
  if (path == MOEQ_PATH_FORWARD_NORM) {
    if (!L->router.q || L->router.rows != d.E) return 0;
    return forward_norm_ws_bytes(to_decode_layer(L, d), d.E, M, K) + kAlign;
  }
  if (path == MOEQ_PATH_GATHER) {
    // any call of up to M tokens: the GEMM form at M, and the light form at
    // the largest token count up to M that takes it
    if (!fits_i32((int64_t)M * K)) return 0;
    const moeq::DecodeLayer dl = to_decode_layer(L, d);
    size_t b = gather_call_ws(dl, M, K, false, nullptr);
    if (light_layer(L, dl)) {
      const int ml = M < light_max_m(dl, K) ? M : light_max_m(dl, K);
      const size_t l = gather_call_ws(dl, ml, K, true, nullptr);
      b = l > b ? l : b;
    }
    return b + kAlign;
  }
  return 0;
}

int qdequant(const moeq_qtensor* W, uint8_t* codes, float* deq, moeq_stream_t stream) {
  int st = check_qt(W, -1, -1, -1);
  if (st) return st;
  if (!codes && !deq) return MOEQ_ERR_NULL_PTR;
  if ((codes && !aligned16(codes)) || (deq && !aligned16(deq))) return MOEQ_ERR_ALIGN;
  moeq::launch_qdequant(to_qt(*W), codes, deq, (hipStream_t)stream);
  return launch_status();
}

int requant_2bit(const moeq_qtensor* W, uint32_t* q_out, uint16_t* s_out, uint16_t* b_out,
                 moeq_stream_t stream) {
  int st = check_qt(W, -1, -1, -1);
  if (st) return st;
  if (W->bits == 2 || is_mx(*W)) return MOEQ_ERR_UNSUPPORTED;   // already 2-bit; not affine
  if (W->group_size == 32) return MOEQ_ERR_BAD_GROUP;   // no 2-bit groups of 32
  if (!q_out || !s_out || !b_out) return MOEQ_ERR_NULL_PTR;
  if (!aligned16(q_out) || !aligned16(s_out) || !aligned16(b_out)) return MOEQ_ERR_ALIGN;
  moeq::launch_requant_2bit(to_qt(*W), q_out, s_out, b_out, (hipStream_t)stream);
  return launch_status();
}

int qmatvec(const moeq_qtensor* W, const float* x, int32_t M, float* y, moeq_stream_t stream) {
  int st = check_qt(W, 1, -1, -1);
  if (st) return st;
  if (M < 0) return MOEQ_ERR_SHAPE;
  if (M == 0) return MOEQ_OK;
  if (!x || !y) return MOEQ_ERR_NULL_PTR;
  if (!fits_i32((int64_t)M * W->cols) || !fits_i32((int64_t)M * W->rows)) return MOEQ_ERR_OVERFLOW;
  if (!aligned16(x) || !aligned16(y)) return MOEQ_ERR_ALIGN;
  moeq::launch_qmatvec(to_qt(*W), x, M, y, (hipStream_t)stream);
  return launch_status();
}

int moe_route(const moeq_qtensor* gate, const float* x_or_logits, int32_t M, int32_t E, int32_t K,
              int32_t renorm, int32_t* topk_idx, float* topk_w, float* logits_out, void* ws,
              size_t ws_bytes, moeq_stream_t stream) {
  if (M < 0 || E <= 0 || E > kMaxE || K < 1 || K > kMaxK || K > E) return MOEQ_ERR_SHAPE;
  if (gate) {
    int st = check_qt(gate, 1, E, -1);
    if (st) return st;
    if (is_mx(*gate)) return MOEQ_ERR_UNSUPPORTED;   // routers are affine
  }
  if (M == 0) return MOEQ_OK;
  if (!x_or_logits || !topk_idx || !topk_w) return MOEQ_ERR_NULL_PTR;
  if (!fits_i32((int64_t)M * E) || !fits_i32((int64_t)M * K) ||
      (gate && !fits_i32((int64_t)M * gate->cols)))
    return MOEQ_ERR_OVERFLOW;
  if (!aligned16(x_or_logits) || !aligned16(topk_idx) || !aligned16(topk_w) ||
      (logits_out && !aligned16(logits_out)))
    return MOEQ_ERR_ALIGN;
  if (gate) {
    if (!ws) return MOEQ_ERR_WORKSPACE;
    if (ws_bytes < moeq::route_ws_bytes(M, E)) return MOEQ_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(ws) % kAlign) return MOEQ_ERR_ALIGN;
  } else if (logits_out) {
    return MOEQ_ERR_UNSUPPORTED;
  }
  moeq::QT g;
  if (gate) g = to_qt(*gate);
  moeq::launch_route(gate ? &g : nullptr, x_or_logits, M, E, K, renorm, topk_idx, topk_w,
                     logits_out, ws, (hipStream_t)stream);
  return launch_status();
}

int moe_expert_forward(const moeq_moe* L, const float* x, const int32_t* topk_idx,
                       const float* topk_w, int32_t M, int32_t K, const float* residual, float* y,
                       void* ws, size_t ws_bytes, moeq_stream_t stream) {
  LayerDims d;
  int st = check_experts(L, &d);
  if (st) return st;
  if (is_mx(L->gate)) return MOEQ_ERR_UNSUPPORTED;   // mxfp4 experts: gather paths only
  if (M < 0 || K < 1 || K > kMaxK || K > d.E) return MOEQ_ERR_SHAPE;
  if (M == 0) return MOEQ_OK;
  if (!x || !topk_idx || !topk_w || !y) return MOEQ_ERR_NULL_PTR;
  if (!fits_i32((int64_t)M * d.H) || !fits_i32((int64_t)M * K * d.I + (int64_t)M * d.Is + M))
    return MOEQ_ERR_OVERFLOW;
  if (!aligned16(x) || !aligned16(topk_idx) || !aligned16(topk_w) || !aligned16(y) ||
      (residual && !aligned16(residual)))
    return MOEQ_ERR_ALIGN;
  const moeq::DecodeLayer dl = to_decode_layer(L, d);
  if (!moeq::decode_supported(dl, K)) return MOEQ_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < expert_ws_bytes(dl, M, K)) return MOEQ_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return MOEQ_ERR_ALIGN;
  st = run_expert_forward(dl, x, topk_idx, topk_w, M, K, residual, y, ws, (hipStream_t)stream);
  if (st) return MOEQ_ERR_UNSUPPORTED;
  return launch_status();
}

int moe_forward(const moeq_moe* L, const float* x, int32_t M, int32_t K, int32_t renorm,
                const float* residual, float* y, int32_t* topk_idx, float* topk_w, void* ws,
                size_t ws_bytes, moeq_stream_t stream) {
  moeq::DecodeLayer dl;
  int32_t E = 0;
  int st = check_forward(L, x, M, K, residual, y, topk_idx, topk_w, &dl, &E);
  if (st != 1) return st;              // an error, or M == 0 (nothing to do)
  if (!ws || ws_bytes < forward_ws_bytes(dl, E, M, K)) return MOEQ_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return MOEQ_ERR_ALIGN;
  return forward_body(L, dl, E, x, M, K, renorm, residual, y, topk_idx, topk_w, ws, (hipStream_t)stream);
}

int moe_forward_noalloc(const moeq_moe* L, const float* x, int32_t M, int32_t K, int32_t renorm,
                        const float* residual, float* y, int32_t* topk_idx, float* topk_w,
                        int32_t* status_out, moeq_stream_t stream) {
  moeq::DecodeLayer dl;
  int32_t E = 0;
  int st = check_forward(L, x, M, K, residual, y, topk_idx, topk_w, &dl, &E);
  if (st != 1) return st;
  if (status_out && !aligned16(status_out)) return MOEQ_ERR_ALIGN;
  const size_t need = forward_ws_bytes(dl, E, M, K);
  if (need > kScratchBytes) return MOEQ_ERR_WORKSPACE;   // beyond the static array
  hipStream_t s = (hipStream_t)stream;
  char* ws = nullptr;
  if ((st = scratch_for_call(dl, L->router, K, need, s, &ws))) return st;
  st = forward_body(L, dl, E, x, M, K, renorm, residual, y, topk_idx, topk_w, ws, s);
  if (st) return st;
  if (status_out) {
    // the call's timeout status out to the caller; a timed-out call leaves
    // the array's counters in an unknown state, so then it is cleared
    moeq::launch_ws_status(ws, status_out, MOEQ_ERR_TIMEOUT, s);
    hipLaunchKernelGGL(k_scratch_clear_if, dim3(kClearBlocks), dim3(256), 0, s, status_out,
                       reinterpret_cast<uint4*>(ws), scratch_used_16(ws));
  }
  return launch_status();
}

int moe_rms_norm(const float* x, int32_t M, int32_t H, const float* norm_w, float eps, float* h,
                 moeq_stream_t stream) {
  if (M < 0 || H <= 0 || H % 4 || bad_eps(eps)) return MOEQ_ERR_SHAPE;
  if (M == 0) return MOEQ_OK;
  if (!x || !norm_w || !h) return MOEQ_ERR_NULL_PTR;
  if (!fits_i32((int64_t)M * H)) return MOEQ_ERR_OVERFLOW;
  if (!aligned16(x) || !aligned16(norm_w) || !aligned16(h)) return MOEQ_ERR_ALIGN;
  moeq::launch_rmsnorm(x, M, H, norm_w, eps, h, (hipStream_t)stream);
  return launch_status();
}

int moe_forward_norm(const moeq_moe* L, const float* x, int32_t M, int32_t K, int32_t renorm,
                     const float* norm_w, float eps, float* y, int32_t* topk_idx, float* topk_w,
                     const float* post_norm_w, float* y_norm, void* ws, size_t ws_bytes,
                     moeq_stream_t stream) {
  LayerDims d;
  int st = check_experts(L, &d);
  if (st) return st;
  if (is_mx(L->gate)) return MOEQ_ERR_UNSUPPORTED;   // mxfp4 experts: gather paths only
  if ((st = check_qt(&L->router, 1, d.E, d.H))) return st;
  if (is_mx(L->router)) return MOEQ_ERR_UNSUPPORTED;
  if (M < 0 || K < 1 || K > kMaxK || K > d.E || bad_eps(eps)) return MOEQ_ERR_SHAPE;
  if (M == 0) return MOEQ_OK;
  if (!x || !norm_w || !y || !topk_idx || !topk_w) return MOEQ_ERR_NULL_PTR;
  if (!post_norm_w != !y_norm) return MOEQ_ERR_NULL_PTR;   // both or neither
  if (y_norm && !aligned16(post_norm_w)) return MOEQ_ERR_ALIGN;
  if (y_norm && !aligned16(y_norm)) return MOEQ_ERR_ALIGN;
  if (!fits_i32((int64_t)M * d.H) || !fits_i32((int64_t)M * d.E) ||
      !fits_i32((int64_t)M * K * d.I + (int64_t)M * d.Is + M))
    return MOEQ_ERR_OVERFLOW;
  if (!aligned16(x) || !aligned16(norm_w) || !aligned16(y) || !aligned16(topk_idx) ||
      !aligned16(topk_w))
    return MOEQ_ERR_ALIGN;
  const moeq::DecodeLayer dl = to_decode_layer(L, d);
  if (!moeq::decode_supported(dl, K)) return MOEQ_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < forward_norm_ws_bytes(dl, d.E, M, K)) return MOEQ_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return MOEQ_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  const QT router = to_qt(L->router);
  if (moeq::fused_supported(dl, router, M, K)) {
    const moeq::RouteIn R{router, renorm, topk_idx, topk_w};
    st = moeq::launch_moe_forward_norm(dl, R, x, M, K, norm_w, eps, y, ws, s);
  } else {
    // normalize into the workspace, route and run the experts on h, add x back
    char* base = reinterpret_cast<char*>(ws);
    float* h = reinterpret_cast<float*>(base + align_up(forward_ws_bytes(dl, d.E, M, K)));
    moeq::launch_rmsnorm(x, M, d.H, norm_w, eps, h, s);
    const moeq::DecState ds = moeq::dec_state(dl, K, base);
    double* l64 = reinterpret_cast<double*>(base + align_up(expert_ws_bytes(dl, M, K)));
    moeq::launch_route_parts(&router, h, M, d.E, K, renorm, topk_idx, topk_w, nullptr, l64,
                             ds.route_ctr, s);
    st = run_expert_forward(dl, h, topk_idx, topk_w, M, K, x, y, base, s);
  }
  if (st) return MOEQ_ERR_UNSUPPORTED;
  // the norm after the combine: the next block's input, from the finished y
  if (y_norm) moeq::launch_rmsnorm(y, M, d.H, post_norm_w, eps, y_norm, s);
  return launch_status();
}

namespace {

// The device-mapped address of pinned host memory [p, p + n), or nullptr when
// either end is not host memory the device can read or the mapping of the
// range is not contiguous.
const char* mapped_host_range(const void* p, uint64_t n) {
  if (!p || n == 0) return nullptr;
  hipPointerAttribute_t a{}, b{};
  const char* last = static_cast<const char*>(p) + (n - 1);
  if (hipPointerGetAttributes(&a, p) != hipSuccess || hipPointerGetAttributes(&b, last) != hipSuccess) {
    (void)hipGetLastError();   // not a registered pointer: leave no error behind
    return nullptr;
  }
  if (a.type != hipMemoryTypeHost || b.type != hipMemoryTypeHost || !a.devicePointer ||
      !b.devicePointer)
    return nullptr;
  const char* da = static_cast<const char*>(a.devicePointer);
  if (static_cast<const char*>(b.devicePointer) - da != (ptrdiff_t)(n - 1)) return nullptr;
  return da;
}

// Host and slot stacks of a slot cache: same shapes except the expert count.
int check_slot_stacks(const moeq_moe* host, const moeq_moe* slots, int S, LayerDims* dh) {
  LayerDims ds;
  int st = check_experts(host, dh);
  if (st) return st;
  if ((st = check_experts(slots, &ds))) return st;
  if (S < 1 || ds.E != S || ds.H != dh->H || ds.I != dh->I) return MOEQ_ERR_SHAPE;
  const moeq_qtensor* hq[3] = {&host->gate, &host->up, &host->down};
  const moeq_qtensor* sq[3] = {&slots->gate, &slots->up, &slots->down};
  for (int i = 0; i < 3; ++i)
    if (hq[i]->bits != sq[i]->bits || hq[i]->group_size != sq[i]->group_size ||
        hq[i]->mode != sq[i]->mode)
      return MOEQ_ERR_SHAPE;
  return MOEQ_OK;
}

}  // namespace

int moe_stream_experts(moeq_slot_cache* C, const int32_t* topk_idx_host, int32_t M, int32_t K,
                       int32_t* slot_idx_host, int32_t* n_copied, moeq_stream_t stream) {
  if (!C) return MOEQ_ERR_NULL_PTR;
  LayerDims dh;
  int st = check_slot_stacks(&C->host, &C->slots, C->n_slots, &dh);
  if (st) return st;
  const int E = dh.E, S = C->n_slots;
  const moeq_qtensor* hq[3] = {&C->host.gate, &C->host.up, &C->host.down};
  const moeq_qtensor* sq[3] = {&C->slots.gate, &C->slots.up, &C->slots.down};
  if (M < 0 || K < 1 || K > kMaxK) return MOEQ_ERR_SHAPE;
  if (n_copied) *n_copied = 0;
  if (M == 0) return MOEQ_OK;
  if (!topk_idx_host || !slot_idx_host || !C->slot_expert || !C->slot_stamp) return MOEQ_ERR_NULL_PTR;
  // the call's distinct experts, in order of first appearance
  std::vector<int> need;
  std::vector<int> where(E, -1);            // expert -> its slot for this call
  for (int64_t i = 0; i < (int64_t)M * K; ++i) {
    const int e = topk_idx_host[i];
    if (e < 0 || e >= E || where[e] == -2) continue;
    where[e] = -2;
    need.push_back(e);
  }
  if ((int)need.size() > S) return MOEQ_ERR_WORKSPACE;
  const int64_t now = ++C->clock;
  // hits keep their slots (and are stamped first, so no miss evicts them)
  for (int s = 0; s < S; ++s) {
    const int e = C->slot_expert[s];
    if (e >= 0 && e < E && where[e] == -2) {
      where[e] = s;
      C->slot_stamp[s] = now;
    }
  }
  int copied = 0;
  for (int e : need) {
    if (where[e] >= 0) continue;
    // an empty slot, else the least recently used one not used by this call
    int v = -1;
    for (int s = 0; s < S; ++s) {
      if (C->slot_stamp[s] == now) continue;
      if (C->slot_expert[s] < 0) { v = s; break; }
      if (v < 0 || C->slot_stamp[s] < C->slot_stamp[v]) v = s;
    }
    if (v < 0) return MOEQ_ERR_WORKSPACE;   // (cannot happen: need.size() <= S)
    for (int i = 0; i < 3; ++i) {
      const moeq_qtensor& h = *hq[i];
      const moeq_qtensor& d = *sq[i];
      const size_t qb = (size_t)h.rows * h.cols / (32 / h.bits) * sizeof(uint32_t);
      const size_t sbytes = (size_t)h.rows * (h.cols / h.group_size) * (is_mx(h) ? 1 : 2);
      hipStream_t st_ = (hipStream_t)stream;
      const char* hqp = reinterpret_cast<const char*>(h.q) + (size_t)e * qb;
      char* dqp = reinterpret_cast<char*>(const_cast<uint32_t*>(d.q)) + (size_t)v * qb;
      if (hipMemcpyAsync(dqp, hqp, qb, hipMemcpyHostToDevice, st_) != hipSuccess) return MOEQ_ERR_LAUNCH;
      const char* hs = reinterpret_cast<const char*>(h.scales) + (size_t)e * sbytes;
      char* ds_ = reinterpret_cast<char*>(const_cast<uint16_t*>(d.scales)) + (size_t)v * sbytes;
      if (hipMemcpyAsync(ds_, hs, sbytes, hipMemcpyHostToDevice, st_) != hipSuccess) return MOEQ_ERR_LAUNCH;
      if (!is_mx(h)) {
        const char* hb = reinterpret_cast<const char*>(h.biases) + (size_t)e * sbytes;
        char* db = reinterpret_cast<char*>(const_cast<uint16_t*>(d.biases)) + (size_t)v * sbytes;
        if (hipMemcpyAsync(db, hb, sbytes, hipMemcpyHostToDevice, st_) != hipSuccess)
          return MOEQ_ERR_LAUNCH;
      }
    }
    C->slot_expert[v] = e;
    C->slot_stamp[v] = now;
    where[e] = v;
    ++copied;
  }
  for (int64_t i = 0; i < (int64_t)M * K; ++i) {
    const int e = topk_idx_host[i];
    slot_idx_host[i] = (e < 0 || e >= E) ? S : where[e];
  }
  if (n_copied) *n_copied = copied;
  return MOEQ_OK;
}

int moe_stream_experts_device(moeq_slot_cache_dev* C, const int32_t* topk_idx, int32_t M, int32_t K,
                              int32_t* slot_idx, int32_t* n_copied, moeq_stream_t stream) {
  if (!C) return MOEQ_ERR_NULL_PTR;
  LayerDims dh;
  const int S = C->n_slots;
  int st = check_slot_stacks(&C->host, &C->slots, S, &dh);
  if (st) return st;
  const int E = dh.E;
  if (M < 0 || K < 1 || K > kMaxK || S > moeq::kMaxStreamSlots || E > moeq::kMaxStreamExperts)
    return MOEQ_ERR_SHAPE;
  if ((int64_t)M * K > S) return MOEQ_ERR_WORKSPACE;
  if (M == 0) return MOEQ_OK;
  if (!topk_idx || !slot_idx || !C->slot_expert || !C->slot_stamp || !C->copy_list)
    return MOEQ_ERR_NULL_PTR;
  if (!aligned16(topk_idx) || !aligned16(slot_idx) || !aligned16(C->slot_expert) ||
      !aligned16(C->slot_stamp) || !aligned16(C->copy_list) || (n_copied && !aligned16(n_copied)))
    return MOEQ_ERR_ALIGN;
  moeq::StreamCopy P{};
  const moeq_qtensor* hq[3] = {&C->host.gate, &C->host.up, &C->host.down};
  const moeq_qtensor* sq[3] = {&C->slots.gate, &C->slots.up, &C->slots.down};
  uint64_t per_expert = 0;
  for (int i = 0; i < 3; ++i) {
    const moeq_qtensor& h = *hq[i];
    const uint64_t qb = (uint64_t)h.rows * h.cols / (32 / h.bits) * sizeof(uint32_t);
    const uint64_t sb = (uint64_t)h.rows * (h.cols / h.group_size) * (is_mx(h) ? 1 : 2);
    const void* hp[3] = {h.q, h.scales, is_mx(h) ? nullptr : h.biases};
    const void* dp[3] = {sq[i]->q, sq[i]->scales, is_mx(h) ? nullptr : sq[i]->biases};
    const uint64_t nb[3] = {qb, sb, sb};
    for (int j = 0; j < 3; ++j) {
      if (!hp[j]) continue;
      const char* src = mapped_host_range(hp[j], nb[j] * E);
      if (!src) return MOEQ_ERR_HOST_MEMORY;
      if (!aligned16(src)) return MOEQ_ERR_ALIGN;
      P.src[P.nseg] = src;
      P.dst[P.nseg] = static_cast<char*>(const_cast<void*>(dp[j]));
      P.bytes[P.nseg] = nb[j];
      ++P.nseg;
      per_expert += nb[j];
    }
  }
  // about 96 KB per block, so a few experts spread over a few hundred blocks
  P.parts = (int)std::min<uint64_t>(256, std::max<uint64_t>(1, per_expert / (96u << 10)));
  if (!fits_i32((int64_t)M * K * P.parts)) return MOEQ_ERR_OVERFLOW;
  if (moeq::launch_stream_experts(P, topk_idx, M * K, E, S, C->slot_expert, C->slot_stamp, slot_idx,
                                  C->copy_list, n_copied, (hipStream_t)stream))
    return MOEQ_ERR_UNSUPPORTED;
  return launch_status();
}

int moe_workspace_status(void* ws, int32_t* status_out, moeq_stream_t stream) {
  if (!ws || !status_out) return MOEQ_ERR_NULL_PTR;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return MOEQ_ERR_ALIGN;
  if (!aligned16(status_out)) return MOEQ_ERR_ALIGN;
  moeq::launch_ws_status(ws, status_out, MOEQ_ERR_TIMEOUT, (hipStream_t)stream);
  return launch_status();
}

int moe_gather_qmm(const moeq_moe* L, const uint16_t* x_bf16, const int32_t* topk_idx,
                   const float* topk_w, int32_t M, int32_t K, float* y, void* ws, size_t ws_bytes,
                   moeq_stream_t stream) {
  LayerDims d;
  int st = check_experts(L, &d);
  if (st) return st;
  if (L->has_shared) return MOEQ_ERR_UNSUPPORTED;
  if (M < 0 || K < 1 || K > kMaxK || K > d.E) return MOEQ_ERR_SHAPE;
  if (M == 0) return MOEQ_OK;
  if (!x_bf16 || !topk_idx || !topk_w || !y) return MOEQ_ERR_NULL_PTR;
  const int64_t n = (int64_t)M * K;
  if (!fits_i32(n) || !fits_i32((int64_t)M * d.H) || !fits_i32(n * d.I) || !fits_i32(n * d.H / 4) ||
      !fits_i32(max_tiles_for((int)n, d.E)))
    return MOEQ_ERR_OVERFLOW;
  if (!aligned16(x_bf16) || !aligned16(topk_idx) || !aligned16(topk_w) || !aligned16(y))
    return MOEQ_ERR_ALIGN;
  const moeq::DecodeLayer dl = to_decode_layer(L, d);
  const bool light = light_gather(L, dl, M, K);
  size_t x_off = 0;
  const size_t need = gather_call_ws(dl, M, K, light, &x_off);
  if (!ws || ws_bytes < need) return MOEQ_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return MOEQ_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  char* base = reinterpret_cast<char*>(ws);
  if (light) {
    float* xf = reinterpret_cast<float*>(base + x_off);
    moeq::launch_bf16_widen(x_bf16, xf, (int64_t)M * d.H, s);
    moeq::BatchWs b;
    batch_ws(base, dl, M, K, &b, gather_counts_bytes(d.E));
    if (moeq::launch_batch_forward(dl, xf, topk_idx, topk_w, M, K, nullptr, y, b, s))
      return MOEQ_ERR_UNSUPPORTED;
    return launch_status();
  }
  moeq::GatherWs g;
  gather_ws(base + moeq::dec_state(dl, K, nullptr).bytes, d.E, (int)n, d.I, d.H, true, &g);
  moeq::launch_sort_pairs(topk_idx, (int)n, d.E, g, s);
  moeq::launch_gemm_gate_up(to_qt(L->gate), to_qt(L->up), x_bf16, K, g, (int)n, s);
  moeq::launch_gemm_down(to_qt(L->down), topk_w, g, (int)n, s);
  moeq::launch_combine(g.ypair, topk_idx, M, K, d.H, d.E, y, s);
  return launch_status();
}

int gather_qmm(const moeq_qtensor* W, const uint16_t* x_bf16, const int32_t* rhs_idx, int32_t n,
               int32_t sorted, float* out, void* ws, size_t ws_bytes, moeq_stream_t stream) {
  int st = check_qt(W, -1, -1, -1);
  if (st) return st;
  if (W->batch > kMaxE) return MOEQ_ERR_SHAPE;
  if (n < 0) return MOEQ_ERR_SHAPE;
  if (n == 0) return MOEQ_OK;
  if (!x_bf16 || !rhs_idx || !out) return MOEQ_ERR_NULL_PTR;
  if (!fits_i32((int64_t)n * W->cols) || !fits_i32((int64_t)n * W->rows) ||
      !fits_i32(max_tiles_for(n, W->batch)))
    return MOEQ_ERR_OVERFLOW;
  if (!aligned16(x_bf16) || !aligned16(rhs_idx) || !aligned16(out)) return MOEQ_ERR_ALIGN;
  moeq::GatherWs g;
  const size_t need = gather_ws(nullptr, W->batch, n, 0, 0, false, nullptr);
  if (!ws || ws_bytes < need) return MOEQ_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return MOEQ_ERR_ALIGN;
  gather_ws(reinterpret_cast<char*>(ws), W->batch, n, 0, 0, false, &g);
  hipStream_t s = (hipStream_t)stream;
  if (sorted)   // rows in place, each expert's run of rows is its tiles
    moeq::launch_runs(rhs_idx, n, W->batch, g, s);
  else
    moeq::launch_sort_pairs(rhs_idx, n, W->batch, g, s);
  moeq::launch_gemm_plain(to_qt(*W), x_bf16, out, g, n, s);
  moeq::launch_mark_invalid_rows(rhs_idx, n, W->batch, W->rows, sorted ? g.offsets : nullptr, out, s);
  return launch_status();
}

}  // extern "C"
