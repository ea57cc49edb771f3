/*
 * moeq.h - C ABI of libmoeq.so: the affine group-quantized mixture-of-experts
 * FFN step on AMD MI355X (gfx950).
 *
 * The step (markbaseengine MOE_ROUTER_WORKS_BREAKTHROUGH, "Forward Pass
 * Sequence"; flash-moe-inference skill page, per-layer pipeline listing):
 *   router projection -> softmax -> top-K -> for each selected expert a fused
 *   dequantize gate/up matvec -> SwiGLU -> down projection -> weighted combine,
 *   with an optional shared expert scaled by a sigmoid gate.
 * The many-token form runs the expert products as gather_qmm (ml-explore/mlx
 * issue #3856, minimal repro: rows sorted by expert, x_i @ deq(W[idx_i])^T).
 *
 * Weight format (danveloper/flash-moe issue thread, quantization config and
 * the 8-bit gate diagnosis; flash-moe-inference skill page, matvec_4bit_fma):
 *   a matrix [rows][cols] ("out" x "in") stores codes of `bits` bits packed
 *   along the input dimension into uint32 words, low bits first: column k is
 *   field k % (32/bits) of word k / (32/bits).  Each group of `group_size`
 *   consecutive input columns has one bf16 scale and one bf16 bias and the
 *   dequantized weight is  w = scale * code + bias.  The bit width is a
 *   property of each tensor (router and shared-expert gates may be 8-bit while
 *   experts are 4-bit).
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller (except the
 *    host arrays and pinned host stacks of moe_stream_experts, documented
 *    there); the library allocates nothing, keeps no global mutable state
 *    besides what lives in the caller's workspace (and slot cache), and only
 *    enqueues work on `stream` (no host sync).
 *  - Every argument is validated on the host BEFORE anything is launched; on
 *    a bad argument the call returns a negative moeq_status and launches
 *    nothing.  A kernel launch failure returns MOEQ_ERR_LAUNCH.
 *  - Shapes are int32 and every derived index fits int32 (checked:
 *    MOEQ_ERR_OVERFLOW); rows, tokens and pairs need not be multiples of any
 *    tile size (ragged tails are computed exactly).
 *  - Device pointers must be 16-byte aligned (MOEQ_ERR_ALIGN).
 *  - Inputs are finite; with NaN/Inf inputs the outputs are unspecified.
 *  - Outputs never alias inputs.
 *  - Workspaces: sized by moe_workspace_size().  A workspace must hold zeros
 *    before its first use (e.g. torch.zeros); every call leaves its counters
 *    at zero again.  The counters sit at offsets that do not depend on M, so
 *    one workspace serves any sequence of calls of its path, for one layer
 *    shape and one K, with any M up to the M it was sized for (the calls of
 *    MOEQ_PATH_DECODE and MOEQ_PATH_FORWARD share one layout).  Calls that
 *    share one workspace must be ordered on one stream; concurrent calls need
 *    separate workspaces.
 */
#ifndef MOEQ_H
#define MOEQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *moeq_stream_t; /* a hipStream_t (NULL = the null stream) */

typedef enum moeq_status {
  MOEQ_OK = 0,
  MOEQ_ERR_NULL_PTR = -1,    /* a required pointer is NULL                      */
  MOEQ_ERR_BAD_BITS = -2,    /* bits not in {2, 4, 8}                           */
  MOEQ_ERR_BAD_GROUP = -3,   /* group_size not 32, 64 or 128 (2 bits: 64 or 128) */
  MOEQ_ERR_K_TAIL = -4,      /* cols not a multiple of group_size               */
  MOEQ_ERR_SHAPE = -5,       /* inconsistent shapes (hidden/inter/experts, top-K) */
  MOEQ_ERR_OVERFLOW = -6,    /* a size or an index would not fit int32          */
  MOEQ_ERR_ALIGN = -7,       /* a device pointer is not 16-byte aligned         */
  MOEQ_ERR_WORKSPACE = -8,   /* workspace missing or smaller than required      */
  MOEQ_ERR_UNSUPPORTED = -9, /* valid request outside what this build computes  */
  MOEQ_ERR_LAUNCH = -10,     /* the HIP runtime rejected a kernel launch        */
  MOEQ_ERR_HOST_MEMORY = -11, /* host memory not pinned and mapped for the device */
  MOEQ_ERR_TIMEOUT = -12     /* a bounded wait inside a decode launch gave up
                                (reported by moe_workspace_status)              */
} moeq_status;

/* One quantized matrix [rows][cols], or a stack of `batch` such matrices laid
 * out back to back (expert e starts at q + e*rows*(cols*bits/32)).
 *   q      : uint32 [batch][rows][cols*bits/32], codes low bits first
 *   scales : bf16 bit patterns [batch][rows][cols/group_size]
 *   biases : bf16 bit patterns, same shape as scales
 * `group_size` is the number of input columns per group (32, 64 or 128; at
 * 2 bits 64 or 128, so that the 64 codes of one 16-byte chunk share a group),
 * not a group count.  cols must be a multiple of it; at group size 32 cols
 * may end on half a 64-column step.  Every expert matrix of a layer (and the
 * shared expert's gate/up/down) uses one group size (MOEQ_ERR_UNSUPPORTED
 * otherwise); the router and the shared expert's gate row may use their own.
 * mode MOEQ_MODE_MXFP4 (the mxfp4 mode the mlx issue runs beside affine; its
 * format is the OCP Microscaling FP4 one): bits 4 and group_size 32
 * (MOEQ_ERR_BAD_BITS / MOEQ_ERR_BAD_GROUP otherwise), 4-bit E2M1 codes
 * packed like affine 4-bit codes (sign, two exponent bits with bias 1, one
 * mantissa bit: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6), one E8M0 scale byte per
 * 32 columns (2^(e - 127); 255 is NaN and gives unspecified outputs), no bias.
 * qdequant, qmatvec, gather_qmm and moe_gather_qmm take it; the decode entry
 * points, moe_route and requant_2bit return MOEQ_ERR_UNSUPPORTED.  Any other
 * mode value: MOEQ_ERR_UNSUPPORTED.
 * The markbaseengine expert kernel hung when this parameter was missing or garbage
 * (MOE_FIX_SUCCESS_EXPERT_WORKS, "Bug Details"), so it is an explicit,
 * validated field here. */
#define MOEQ_MODE_AFFINE 0  /* w = scale * code + bias, bf16 scale and bias per group */
#define MOEQ_MODE_MXFP4 1   /* w = e2m1(code) * 2^(e - 127), one E8M0 byte e per 32 cols */

typedef struct moeq_qtensor {
  const uint32_t *q;
  const uint16_t *scales;   /* MOEQ_MODE_MXFP4: uint8 E8M0 bytes [batch][rows][cols/32] */
  const uint16_t *biases;   /* MOEQ_MODE_MXFP4: unused, may be NULL */
  int32_t batch;
  int32_t rows;
  int32_t cols;
  int32_t bits;
  int32_t group_size;
  int32_t mode;             /* MOEQ_MODE_AFFINE (0) or MOEQ_MODE_MXFP4 (1) */
} moeq_qtensor;

/* One MoE layer.  router [1][E][H]; gate, up [E][I][H]; down [E][H][I].
 * has_shared != 0 adds a shared expert: sh_gate, sh_up [1][Is][H],
 * sh_down [1][H][Is] and the one-row shared_expert_gate [1][1][H], whose
 * sigmoid scales the shared expert's output (flash-moe-inference skill page,
 * moe_combine_residual: combine + residual + sigmoid gate). */
typedef struct moeq_moe {
  moeq_qtensor router;
  moeq_qtensor gate;
  moeq_qtensor up;
  moeq_qtensor down;
  int32_t has_shared;
  moeq_qtensor sh_gate;
  moeq_qtensor sh_up;
  moeq_qtensor sh_down;
  moeq_qtensor sh_expert_gate;
} moeq_moe;

/* Experts held in host memory and streamed into device slots (the models
 * larger than HBM case): caller-owned memory, contents managed by
 * moe_stream_experts.
 *   host  : gate, up, down stacks [E][...] in PINNED host memory
 *           (hipHostMalloc; pageable memory works but the copies then
 *           serialize with the host); the other fields are unused
 *   slots : gate, up, down stacks [S][...] in device memory, the same
 *           per-expert shapes, bits, group size and mode as host
 *   slot_expert : host int32 [S], the expert each slot holds, -1 = empty
 *                 (the caller sets every entry to -1 before the first call)
 *   slot_stamp  : host int64 [S], the last call that used each slot
 *   clock       : host counter of calls (start at 0)
 *   n_slots     : S */
typedef struct moeq_slot_cache {
  moeq_moe host;
  moeq_moe slots;
  int32_t *slot_expert;
  int64_t *slot_stamp;
  int64_t clock;
  int32_t n_slots;
} moeq_slot_cache;

/* The device-side form of the slot cache (moe_stream_experts_device): the
 * same host and slot stacks, the LRU state in device memory.
 *   host        : expert stacks [E] in pinned host memory that the device can
 *                 read (hipHostMalloc, torch pin_memory); biases NULL for mxfp4
 *   slots       : the same stacks with S experts, in device memory
 *   slot_expert : DEVICE int32 [S], the expert each slot holds, -1 = empty
 *                 (the caller fills it with -1 once)
 *   slot_stamp  : DEVICE int64 [S + 1], the call that last used each slot;
 *                 element S counts the calls (the caller zeroes it once)
 *   copy_list   : DEVICE int32 [2 S + 1], scratch of one call (the copies)
 *   n_slots     : S, 1 <= S <= 1024
 * The state arrays belong to the library between calls. */
typedef struct moeq_slot_cache_dev {
  moeq_moe host;
  moeq_moe slots;
  int32_t *slot_expert;
  int64_t *slot_stamp;
  int32_t *copy_list;
  int32_t n_slots;
} moeq_slot_cache_dev;

/* Workspace paths for moe_workspace_size(). */
#define MOEQ_PATH_ROUTE 0   /* moe_route                                   */
#define MOEQ_PATH_DECODE 1  /* moe_expert_forward                          */
#define MOEQ_PATH_GATHER 2  /* moe_gather_qmm                              */
#define MOEQ_PATH_GQMM 3    /* gather_qmm (single projection; K is unused) */
#define MOEQ_PATH_FORWARD 4 /* moe_forward                                 */
#define MOEQ_PATH_FORWARD_NORM 5 /* moe_forward_norm                       */

/* Human-readable text for a status code (static storage). */
const char *moeq_status_string(int status);

/* Library version string (static storage). */
const char *moeq_version(void);

/* Workspace bytes needed by the given path for a layer, M tokens and top-K.
 * For MOEQ_PATH_GQMM pass the stacked weight as L->gate and n rows as M.
 * Returns 0 when the arguments are invalid. */
size_t moe_workspace_size(const moeq_moe *L, int32_t M, int32_t K, int32_t path);

/* qdequant: unpack and dequantize a whole (stacked) quantized tensor.
 *   codes : nullable, uint8 [batch][rows][cols], the integer codes
 *   deq   : nullable, fp32  [batch][rows][cols], fp32(scale*code + bias)
 * Defines: the unpack / dequantize step itself (flash-moe-inference,
 * matvec_4bit_fma: (nibble*scale + bias)).  Both outputs are exact: the
 * bf16*code product is exact in fp32, so deq is the single rounding of
 * scale*code + bias. */
int qdequant(const moeq_qtensor *W, uint8_t *codes, float *deq, moeq_stream_t stream);

/* qmatvec: y[m][r] = sum_k deq(W)[r][k] * x[m][k]  (fp32 in, fp32 out, fp32
 * accumulation) for one matrix (W->batch == 1), M >= 1 tokens.
 *   x : fp32 [M][cols];  y : fp32 [M][rows]
 * Defines: the dequantizing matrix-vector product of the flash-moe
 * matvec_4bit_fma sketch (weights, scales, biases, x, out) with explicit
 * in/out dimensions and group parameter (markbaseengine expert kernel). */
int qmatvec(const moeq_qtensor *W, const float *x, int32_t M, float *y,
            moeq_stream_t stream);

/* moe_route: router projection, softmax over all E experts, top-K by
 * (score descending, index ascending), weights p[idx] / sum(p[idx]) when
 * renorm != 0, else p[idx].
 *   gate      : the router [1][E][H]; NULL selects logits-in mode, where
 *               x_or_logits holds fp32 logits [M][E]
 *   x_or_logits : fp32 [M][H] activations (or [M][E] logits)
 *   topk_idx  : int32 [M][K] out, in selection order
 *   topk_w    : fp32  [M][K] out
 *   logits_out: nullable fp32 [M][E] out (router mode only)
 *   ws        : workspace of moe_workspace_size(L, M, K, MOEQ_PATH_ROUTE)
 * The router logits are accumulated in fp64 on the GPU so the top-K decision
 * is taken on fp64 values.  1 <= K <= min(E, 16), E <= 1024.
 * Defines: "Forward Pass Sequence" steps 1-4 (markbaseengine) and "softmax +
 * topK routing" (flash-moe pipeline), kept on the device. */
int moe_route(const moeq_qtensor *gate, const float *x_or_logits, int32_t M, int32_t E,
              int32_t K, int32_t renorm, int32_t *topk_idx, float *topk_w,
              float *logits_out, void *ws, size_t ws_bytes, moeq_stream_t stream);

/* moe_expert_forward: the expert part of the step for fp32 activations
 * (decode, any M >= 1):
 *   y[t] = sum_{k<K} topk_w[t][k] * down_e(silu(gate_e x_t) * up_e x_t),
 *          e = topk_idx[t][k]
 *        + sigmoid(sh_expert_gate . x_t) * FFN_shared(x_t)   (if has_shared)
 *        + residual[t]                                          (if non-NULL)
 * with fp32 accumulation; the K terms are added in slot order, so results are
 * bitwise reproducible run to run.
 *   x : fp32 [M][H];  topk_idx int32 [M][K] (each in [0, E));  topk_w fp32 [M][K]
 *   residual : nullable fp32 [M][H];  y : fp32 [M][H]
 * Defines: "Forward Pass Sequence" step 5-6 (markbaseengine), flash-moe swiglu
 * and moe_combine_residual sketches. */
int moe_expert_forward(const moeq_moe *L, const float *x, const int32_t *topk_idx,
                       const float *topk_w, int32_t M, int32_t K, const float *residual,
                       float *y, void *ws, size_t ws_bytes, moeq_stream_t stream);

/* moe_forward: the whole step for fp32 activations (decode): moe_route on
 * L->router (router mode) followed by moe_expert_forward, with the same
 * results as that pair of calls.
 *   x : fp32 [M][H];  renorm as in moe_route;  residual : nullable fp32 [M][H]
 *   y : fp32 [M][H] out;  topk_idx int32 [M][K] and topk_w fp32 [M][K] out
 *   ws : workspace of moe_workspace_size(L, M, K, MOEQ_PATH_FORWARD)
 * With an 8-bit router and M <= 4 the whole step is ONE launch: the router
 * rows, the top-K selection and the experts run in one grid, the expert units
 * starting their weight loads as soon as the selection is published, so the
 * routing round trip through the host or a second launch disappears; other
 * cases run the two launches.
 * Defines: the per-layer pipeline of the flash-moe skill page (router
 * projection, softmax + topK, expert forward, combine) and the markbaseengine
 * "Forward Pass Sequence", kept on the device. */
int moe_forward(const moeq_moe *L, const float *x, int32_t M, int32_t K, int32_t renorm,
                const float *residual, float *y, int32_t *topk_idx, float *topk_w, void *ws,
                size_t ws_bytes, moeq_stream_t stream);

/* moe_forward_noalloc: moe_forward with no workspace argument and no
 * allocation, for callers that cannot allocate device memory around the
 * call (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments and results as moe_forward; the
 * workspace is a static device array of the library, 16 MiB on each device,
 * held from the library's first use on that device until the process ends.
 *   status_out : nullable device int32 [2], 16-byte aligned: after the call,
 *                as moe_workspace_status reports for moe_forward's workspace
 *                ([0] MOEQ_OK or MOEQ_ERR_TIMEOUT, [1] the raw bits); a call
 *                that reports a timeout also clears the array, so the next
 *                call starts clean
 * Returns MOEQ_ERR_WORKSPACE when the call needs more than the array holds
 * (moe_workspace_size(L, M, K, MOEQ_PATH_FORWARD) > 16 MiB: e.g. more than
 * about 64 tokens at the 397B-A17B shapes), before anything is launched.
 * Every call on a device shares that device's array, which keeps the last
 * call's state: a call whose layer shape or K differs from the previous
 * call's clears the array first with a fill kernel on `stream`.  Calls on one
 * device must therefore be ordered (one stream, or streams the caller
 * synchronizes); calls that overlap on one device race and give wrong
 * results.  Calls no hipMalloc, hipFree or allocating library routine. */
int moe_forward_noalloc(const moeq_moe *L, const float *x, int32_t M, int32_t K, int32_t renorm,
                        const float *residual, float *y, int32_t *topk_idx, float *topk_w,
                        int32_t *status_out, moeq_stream_t stream);

/* moe_rms_norm: h[m] = x[m] / sqrt(mean_k(x[m][k]^2) + eps) * norm_w, per row.
 *   x : fp32 [M][H];  norm_w : fp32 [H];  h : fp32 [M][H] out;  H % 4 == 0;
 *   eps >= 0 and finite (MOEQ_ERR_SHAPE otherwise)
 * The mean square is reduced in fp32, its reciprocal square root taken in
 * fp64.
 * Defines: the two-pass RMSNorm before the router (flash-moe-inference skill
 * page, rms_norm_pass1/2: sum of squares, then scale; the CMD2 chain o_proj ->
 * residual_add -> rms_norm -> routing gate of the flash-moe issue thread). */
int moe_rms_norm(const float *x, int32_t M, int32_t H, const float *norm_w, float eps, float *h,
                 moeq_stream_t stream);

/* moe_forward_norm: the step with its neighbours fused, for fp32 decode
 * activations:  h = rms_norm(x), route and run the experts on h, and add the
 * raw row back in the combine:  y = x + MoE(h).  Same results as moe_rms_norm
 * followed by moe_forward(h, residual = x).
 *   x : fp32 [M][H] (the residual stream);  norm_w, eps as in moe_rms_norm
 *   y, topk_idx, topk_w out as in moe_forward
 *   post_norm_w, y_norm : both NULL, or fp32 [H] and fp32 [M][H] out (not
 *               overlapping y): the norm after the combine, y_norm =
 *               rms_norm(y) * post_norm_w with the same eps (the next block's
 *               input), one more launch after the step; NULL for only one of
 *               them is MOEQ_ERR_NULL_PTR
 *   ws : workspace of moe_workspace_size(L, M, K, MOEQ_PATH_FORWARD_NORM)
 * With an 8-bit router and M <= 4 this is ONE launch: every router and
 * gate/up unit stages x * norm_w, reduces the row's mean square itself and
 * scales its finished sums by the reciprocal root (both are linear in the
 * row); otherwise the norm is a launch of its own in front of moe_forward's
 * two launches, h kept in the workspace.
 * Defines: the CMD2/CMD3 chain of the flash-moe-inference skill page (norm,
 * routing, expert forward, combine + residual: moe_combine_residual, then
 * the norm that closes CMD3). */
int moe_forward_norm(const moeq_moe *L, const float *x, int32_t M, int32_t K, int32_t renorm,
                     const float *norm_w, float eps, float *y, int32_t *topk_idx, float *topk_w,
                     const float *post_norm_w, float *y_norm, void *ws, size_t ws_bytes,
                     moeq_stream_t stream);

/* moe_workspace_status: report, then clear, the error word of a decode-family
 * workspace (one sized for MOEQ_PATH_DECODE, MOEQ_PATH_FORWARD or
 * MOEQ_PATH_FORWARD_NORM).
 * The decode launches of moe_expert_forward, moe_forward and moe_forward_norm
 * hand data from one workgroup of the grid to another (routing result, h,
 * the shared gate); every such wait is bounded, and one that runs out of spins
 * gives up instead of hanging the GPU and sets a bit in this word.  The calls
 * whose waits gave up have wrong outputs, and the word stays set until this
 * call clears it.
 *   ws         : the workspace (device, 256-byte aligned)
 *   status_out : device int32 [2], 16-byte aligned: [0] = MOEQ_OK or
 *                MOEQ_ERR_TIMEOUT, [1] = the raw bits (1 ready flag, 2 routing
 *                result, 4 router logits or the slots' expert and weight
 *                pairs, 8 h or shared gate)
 * One small kernel on `stream`, ordered after the work queued before it (no
 * memset node: the call can be captured in a graph).  The host return value
 * only says whether that kernel was queued; the status itself is in
 * status_out once the stream reaches it.  Workspaces of the other paths hold
 * no error word: do not pass them.
 * Defines: no passage of the pages; it reports the bounded cross-workgroup
 * waits this library uses in place of the pages' one-command-buffer-per-stage
 * pipeline (flash-moe-inference skill page, per-layer pipeline). */
int moe_workspace_status(void *ws, int32_t *status_out, moeq_stream_t stream);

/* moe_gather_qmm: the expert part for many bf16 tokens (prefill).  Pairs
 * (token, slot) are sorted by expert on the device; per expert the gathered
 * rows run through a bf16 MFMA gate/up GEMM with a SwiGLU epilogue (h kept in
 * bf16) and a down GEMM scaled by the routing weight; each token then sums its
 * K pairs in slot order.  fp32 output; any M >= 1 (no tile-size alignment).
 * With few rows per expert (M * K <= 4 E, affine experts, layer shapes the
 * batched decode supports) the MFMA tiles would hold a handful of rows, so
 * the call instead streams each touched expert once per tile of two pairs
 * through the batched decode kernels, the activations widened exactly to
 * fp32 (fp32 accumulation throughout; same outputs to within the tolerance,
 * same invalid-index NaN rows).  The workspace of moe_workspace_size covers
 * both forms for every M up to the one it was sized for.
 *   x_bf16 : bf16 bit patterns [M][H];  topk_idx, topk_w as above;  y : fp32 [M][H]
 * has_shared must be 0 (MOEQ_ERR_UNSUPPORTED otherwise).
 * Defines: mlx-lm SwitchGLU through gather_qmm with sorted indices
 * (ml-explore/mlx issue #3856), with exact handling of ragged row counts. */
int moe_gather_qmm(const moeq_moe *L, const uint16_t *x_bf16, const int32_t *topk_idx,
                   const float *topk_w, int32_t M, int32_t K, float *y, void *ws,
                   size_t ws_bytes, moeq_stream_t stream);

/* gather_qmm: one projection per row, the weight picked per row:
 *   out[i] = x[i] @ deq(W[rhs_idx[i]])^T       (transpose=True)
 *   W : stacked [E][N][Kd];  x_bf16 : bf16 [n][Kd];  rhs_idx : int32 [n] in [0, E)
 *   sorted : nonzero if rhs_idx is non-decreasing: the rows are then used in
 *            place with no sort, expert e taking the run of rows that holds
 *            index e; a row outside the run of its own index (indices that
 *            were not in fact non-decreasing) comes out NaN.  0: the rows are
 *            grouped by expert on the device first.
 *   out : fp32 [n][N]; rows whose index is outside [0, E) come out NaN
 * Defines: mx.gather_qmm(x, w, scales, biases, rhs_indices, transpose=True,
 * sorted_indices) of the ml-explore/mlx issue #3856 minimal repro. */
int gather_qmm(const moeq_qtensor *W, const uint16_t *x_bf16, const int32_t *rhs_idx,
               int32_t n, int32_t sorted, float *out, void *ws, size_t ws_bytes,
               moeq_stream_t stream);

/* requant_2bit: requantize a 4- or 8-bit tensor (or stack) to 2 bits per
 * group, keeping the group size (64 or 128).
 *   W       : the source, bits 4 or 8 (2: MOEQ_ERR_UNSUPPORTED), group size
 *             64 or 128 (32: MOEQ_ERR_BAD_GROUP)
 *   q_out   : uint32 [batch][rows][cols/16], 2-bit codes low bits first
 *   s_out, b_out : bf16 bit patterns [batch][rows][cols/group_size]
 *   (all 16-byte aligned, caller-owned, not overlapping the source)
 * Per group of the source, with w = scale*code + bias taken exactly: the
 * 2-bit grid runs from the group's smallest weight lo to its largest hi in
 * three equal steps; each weight gets the nearest grid point's code, ties to
 * the even code, and every code is 0 when hi == lo; s_out = (hi - lo)/3 and
 * b_out = lo, each rounded once to bf16 (nearest, ties to even).  Bit-exact:
 * the codes are integer decisions and the two stored values are exactly
 * rounded.
 * Defines: the 4-bit to 2-bit conversion of the experts
 * (flash-moe-inference skill page, setup steps and the repository layout's
 * repack_experts_2bit.py; the page names the tool, the grid above is the
 * reading taken). */
int requant_2bit(const moeq_qtensor *W, uint32_t *q_out, uint16_t *s_out, uint16_t *b_out,
                 moeq_stream_t stream);

/* moe_stream_experts: bring the experts a routing result selects into device
 * slots and rewrite the indices to slot numbers, so that moe_expert_forward
 * on a layer whose gate/up/down are C->slots (and whose shared expert, if
 * any, is resident) computes the step for experts that live in host memory.
 *   topk_idx_host : host int32 [M][K] (e.g. moe_route's output copied back)
 *   slot_idx_host : host int32 [M][K] out: the slot of each pair; an index
 *                   outside [0, E) maps to slot S (its row then comes out NaN,
 *                   as with any out-of-range index)
 *   n_copied      : nullable host int32 out: experts copied by this call
 * The distinct experts of the call stay in their slots if already there
 * (least recently used slots are refilled first); each missing expert's
 * codes, scales and biases go out as hipMemcpyAsync host->device copies on
 * `stream`, in order with the caller's other work there: a slot is only
 * refilled after the work queued before it on that stream (the previous
 * forward that read it).  More distinct experts than slots:
 * MOEQ_ERR_WORKSPACE, nothing copied.  Runs on the host; returns once the
 * copies are queued.
 * Defines: the K parallel expert reads per layer into expert buffers, the OS
 * page cache acting as the LRU (flash-moe-inference skill page, parallel
 * expert loading; the per-layer pipeline's I/O phase), with host memory in
 * place of the SSD and HBM slots in place of the buffers. */
int moe_stream_experts(moeq_slot_cache *C, const int32_t *topk_idx_host, int32_t M, int32_t K,
                       int32_t *slot_idx_host, int32_t *n_copied, moeq_stream_t stream);

/* moe_stream_experts_device: moe_stream_experts with the routing result, the
 * slot choice and the copies all on the device: no host round trip between
 * moe_route and moe_expert_forward, so a layer's route -> stream -> forward
 * chain queues without a synchronization (and can be captured in a graph).
 *   topk_idx : device int32 [M][K] (moe_route's output)
 *   slot_idx : device int32 [M][K] out, the slot of each pair (S for an index
 *              outside [0, E), whose row then comes out NaN)
 *   n_copied : nullable device int32 out, experts copied by this call
 * Two launches on `stream`: one wave takes the LRU decisions of
 * moe_stream_experts (same order, same slots for the same call sequence) and
 * writes the copy list; then one kernel copies every listed expert's codes,
 * scales and biases, its waves reading the pinned host stacks over PCIe.
 * A slot is refilled only after the work queued before it on the stream.
 * M*K must not exceed S (MOEQ_ERR_WORKSPACE), so every call has slots enough
 * whatever it selects; E <= 1024.  Each host stack must be pinned and mapped
 * for the device over its whole extent (checked at its first and last byte:
 * MOEQ_ERR_HOST_MEMORY otherwise).  All other pointers are device pointers,
 * 16-byte aligned.
 * Defines: as moe_stream_experts (flash-moe-inference skill page, parallel
 * expert loading), with the I/O phase issued by the device itself. */
int moe_stream_experts_device(moeq_slot_cache_dev *C, const int32_t *topk_idx, int32_t M, int32_t K,
                              int32_t *slot_idx, int32_t *n_copied, moeq_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEQ_H */
