// Gather GEMMs of the prefill path on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16).
//
// ml-explore/mlx issue #3856 (minimal repro: gather_qmm with rhs_indices,
// transpose=True) defines the product; its row-count defect is why every tile
// here carries its exact row count in int32, rows past it are zero-filled on
// load and never stored.
//
// A block computes a 256-row x 256-column tile of one expert: 256 rows
// gathered through the sorted pair list, 256 weight rows ("B columns").  Per
// 64-wide reduction step (one quantization group) the A rows are staged as
// bf16 in LDS and the B codes dequantized to bf16 in LDS (w = scale*code +
// bias, rounded to nearest even).  LDS holds two stages: while the waves run
// the MFMAs of one stage, the next steps' global loads land in registers (two
// steps ahead), and the step after this one is dequantized and written to
// the other stage a quarter per 16-wide k slice, between the slices' MFMAs
// (affine codes; the mxfp4 form writes the whole stage after the MFMAs), one
// barrier per step.
// Eight waves, two per SIMD, each own a 128x64 sub-tile (4x2 MFMA 32x32
// tiles): the two waves of a SIMD hide each other's load, LDS and barrier
// waits, and a 256-column block re-reads the gathered A rows half as often as
// a 128-column one.
//
// Tile order is XCD-aware: workgroups are dealt round-robin to the 8 XCDs, so
// block b works on item (b % 8) * ceil(T/8) + b / 8 of the T (m-tile, n-tile)
// items in m-major order: all n-tiles of an m-tile run on one XCD back to back
// and the gathered A rows are re-read from that XCD's L2, not from HBM.
//
// Modes: 0 plain   out[pair][n] = x[pair] . W_e[n]                 (fp32)
//        1 gate/up h[sorted row][i] = silu(x.G_e[i]) * (x.U_e[i])  (bf16);
//                  a block's columns are 128 rows i of gate and the same
//                  128 of up (per wave: 32 of each)
//        2 down    ypair[pair][n] = w_pair * (h[sorted row] . D_e[n]) (bf16)
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moeq {

typedef short bf16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// staging registers as a native vector (HIP's uint4 is a struct with a union,
// which keeps the compiler from promoting arrays of it to registers here)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = kGemmBM;  // 256 rows
constexpr int kBN = 256;      // B columns per block
constexpr int kBK = 64;       // one group per k-step
constexpr int kLds = kBK + 8; // padded row stride (bf16 elements): 144 B, conflict-free b128 reads
constexpr int kThreads = 512;   // eight waves, two per SIMD
constexpr int kXcd = 8;
constexpr int kStage = (kBM + kBN) * kLds;                      // bf16 elements per LDS stage
constexpr size_t kGemmLds = 2 * (size_t)kStage * sizeof(uint16_t);

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};   // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// dequantize codes [32h, 32h + 32) of one group (its 16 / 8 / 4 words in v)
// to 16 packed bf16 pairs
template <int BITS>
__device__ __forceinline__ void dequant32h(const u32x4* v, int h, float s, float b, uint32_t* out) {
  constexpr int kPer = 32 / BITS;
  constexpr uint32_t kMask = (1u << BITS) - 1u;
#pragma unroll
  for (int w = 0; w < 32 / kPer; ++w) {
    const int wi = h * (32 / kPer) + w;
    const uint32_t x = v[wi / 4][wi % 4];
#pragma unroll
    for (int j = 0; j < kPer; j += 2)
      out[(w * kPer + j) / 2] = pack_bf16(fmaf(s, (float)((x >> (BITS * j)) & kMask), b),
                                          fmaf(s, (float)((x >> (BITS * j + BITS)) & kMask), b));
  }
}

// mxfp4: the 32 E2M1 codes of one group (4 words) times the group's E8M0
// scale, to 16 packed bf16 pairs, by the scaled conversion instruction (it
// takes the exponent field of s: s = 2^(e-127) as fp32 bits, e = 0 as the
// subnormal 2^-127).  s == 0 marks a masked half step: the codes are cleared
// (the instruction does not scale by zero).
__device__ __forceinline__ void dequant32_mx(const u32x4* v, float s, uint32_t* out) {
  const uint32_t keep = s != 0.f ? 0xFFFFFFFFu : 0u;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t x = v[0][w] & keep;
    out[4 * w + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, s, 0));
    out[4 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, s, 1));
    out[4 * w + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, s, 2));
    out[4 * w + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, s, 3));
  }
}

// E8M0 byte -> the fp32 whose exponent field the conversion reads
__device__ __forceinline__ float e8m0_f32(uint32_t e) {
  return __uint_as_float(e == 0 ? 0x00400000u : e << 23);
}

template <int BITS, int MODE, bool MX = false>
__global__ void __launch_bounds__(kThreads, 1) k_gqmm(QT W, QT W2, int N, int Kd,
                                                      const uint16_t* __restrict__ A, int a_div,
                                                      GatherWs ws, const float* __restrict__ wts,
                                                      void* __restrict__ out, int ntn) {
  extern __shared__ __attribute__((aligned(16))) uint16_t gsm[];
  __shared__ int s_pair[kBM];
  __shared__ float s_w[kBM];
  constexpr int kWords = 64 * BITS / 32;     // code words per group and column
  constexpr int kV = (kWords / 2 + 3) / 4;   // 16-byte words per thread (half a group)

  // ---- XCD-aware item: block b -> item (b % 8) * ceil(T/8) + b / 8
  const int T = ws.n_tiles[0] * ntn;
  const int per = (T + kXcd - 1) / kXcd;
  const int item = (blockIdx.x % kXcd) * per + blockIdx.x / kXcd;
  if (blockIdx.x / kXcd >= per || item >= T) return;
  const int tile = item / ntn;
  const int nt = item - tile * ntn;
  const int4 Tl = ws.tiles[tile];
  const int e = Tl.x, row0 = Tl.y, rows = Tl.z;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int wm = wid & 1, wn = wid >> 1;      // 2 row halves x 4 column quarters

  for (int r = tid; r < kBM; r += kThreads) {
    const int pair = r < rows ? ws.sorted[row0 + r] : 0;
    s_pair[r] = pair;
    if (MODE == 2) s_w[r] = r < rows ? wts[pair] : 0.f;
  }
  __syncthreads();

  // ---- A source rows: rows (tid>>3) + 64u (u < 4), 16-byte segment tid&7
  const int aseg = tid & 7;
  // (32-bit element offsets from A: the activations of one call stay below
  // 2^31 elements).  Rows past the tile's count re-read its first row: an
  // output row depends on its own A row only, and those rows are never stored,
  // so the loads need no branches.
  int aoff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = (tid >> 3) + 64 * u;
    const int rc = r < rows ? r : 0;
    aoff[u] = (MODE == 2 ? row0 + rc : s_pair[rc] / a_div) * Kd;
  }

  // ---- B column of this thread: bc = tid >> 1, codes [32 bh, 32 bh + 32) of
  // each group.  Columns past N read column N-1 (their outputs are never
  // stored).
  const int bc = tid >> 1, bh = tid & 1;
  const uint32_t* bq;
  const uint16_t *bs = nullptr, *bb = nullptr;
  const uint8_t* bs8 = nullptr;                    // mxfp4: E8M0 scale bytes of the column
  int gsz;                                         // elements per group of this column's matrix
  {
    int n;
    const QT* M = &W;
    if (MODE == 1) {
      // wave column cw = bc >> 6 holds gate rows then up rows of i in [32 cw, 32 cw + 32)
      const int cw = bc >> 6, hf = (bc >> 5) & 1;
      n = nt * 128 + cw * 32 + (bc & 31);
      if (hf) M = &W2;
    } else {
      n = nt * kBN + bc;
    }
    const size_t row = (size_t)e * N + min(n, N - 1);
    bq = M->q + row * (Kd / (32 / BITS));
    if constexpr (MX) {
      bs8 = reinterpret_cast<const uint8_t*>(M->scales) + row * (Kd / 32);
    } else {
      bs = M->scales + row * (Kd / M->group_size);
      bb = M->biases + row * (Kd / M->group_size);
    }
    gsz = M->group_size;
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // two register stages of global loads: step k's data lands in stage k % 2
  // (scale and bias stay raw bits until the stage is written to LDS, so the
  // first use of every loaded register is two steps after its load)
  u32x4 a0[4], a1[4], b0[kV], b1[kV];
  uint32_t s0 = 0u, c0 = 0u, s1 = 0u, c1 = 0u;   // raw scale, bias bits
  float m0 = 0.f, m1 = 0.f;                      // 1, or 0 for a masked half step
  // k-steps of 64 columns; Kd may end on half a step (group size 32, an odd
  // number of groups): the missing half is read from valid columns and
  // weighted by zero scale and bias
  const int ksteps = (Kd + kBK - 1) / kBK;

#define MOEQ_GLOAD(AR, BR, SV, CV, MV, KT)                                                    \
  do {                                                                                        \
    const int k_ = (KT);                                                                      \
    const int ac_ = min(k_ * kBK + aseg * 8, Kd - 8);                                         \
    _Pragma("unroll") for (int u = 0; u < 4; ++u)                                             \
      AR[u] = *reinterpret_cast<const u32x4*>(A + aoff[u] + ac_);                             \
    const int cc_ = k_ * kBK + bh * 32;            /* this thread's 32 codes */                \
    const bool ok_ = cc_ < Kd;                                                                \
    const int cv_ = ok_ ? cc_ : cc_ - 32;                                                     \
    const uint32_t* p_ = bq + (size_t)cv_ * BITS / 32;                                        \
    if constexpr (BITS == 2) {                                                                \
      const uint2 t_ = *reinterpret_cast<const uint2*>(p_);                                   \
      BR[0] = u32x4{t_.x, t_.y, 0u, 0u};                                                      \
    } else {                                                                                  \
      _Pragma("unroll") for (int q = 0; q < kV; ++q) BR[q] = reinterpret_cast<const u32x4*>(p_)[q]; \
    }                                                                                         \
    MV = ok_ ? 1.f : 0.f;                          /* loads stay unconditional */              \
    if constexpr (MX) {                            /* one group of 32: scale byte cv_ / 32 */  \
      SV = bs8[cv_ >> 5];                                                                     \
      CV = 0u;                                                                                \
    } else {                                                                                  \
      SV = bs[group_of(cv_, gsz)];                                                            \
      CV = bb[group_of(cv_, gsz)];                                                            \
    }                                                                                         \
  } while (0)
  // MV: the stage's mask (the half-step tail and, for the unused half of the
  // last pair of steps, zero)
#define MOEQ_LSTORE(AR, BR, SRAW, CRAW, MV, BUF)                                              \
  do {                                                                                        \
    const float SV = (MX ? e8m0_f32(SRAW) : bf16_to_f32(SRAW)) * (MV);                        \
    const float CV = (MX ? 0.f : bf16_to_f32(CRAW)) * (MV);                                   \
    uint16_t* As_ = gsm + (BUF) * kStage;                                                     \
    uint16_t* Bs_ = As_ + kBM * kLds;                                                         \
    _Pragma("unroll") for (int u = 0; u < 4; ++u)                                             \
      *reinterpret_cast<u32x4*>(&As_[((tid >> 3) + 64 * u) * kLds + aseg * 8]) = AR[u];       \
    u32x4* d_ = reinterpret_cast<u32x4*>(&Bs_[bc * kLds + bh * 32]);                          \
    uint32_t pk_[16];                                                                         \
    if constexpr (MX) dequant32_mx(BR, SV, pk_);                                              \
    else dequant32h<BITS>(BR, 0, SV, CV, pk_);                                                \
    _Pragma("unroll") for (int q = 0; q < 4; ++q)                                             \
      d_[q] = u32x4{pk_[4 * q], pk_[4 * q + 1], pk_[4 * q + 2], pk_[4 * q + 3]};              \
  } while (0)

  auto mfma_step = [&](int buf) {
    const uint16_t* As = gsm + buf * kStage;
    const uint16_t* Bs = As + kBM * kLds;
    // 4 k16 steps x (4 x 4) tiles
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int kof = kk * 16 + 8 * (lane >> 5);
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        af[mi] = *reinterpret_cast<const bf16x8*>(&As[(wm * 128 + mi * 32 + (lane & 31)) * kLds + kof]);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bfr[ni] = *reinterpret_cast<const bf16x8*>(&Bs[(wn * 64 + ni * 32 + (lane & 31)) * kLds + kof]);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          // the transposed product (weights x activations): the accumulator's
          // lanes run over tokens and its registers over output columns
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ni], af[mi], acc[mi][ni], 0, 0, 0);
    }
  };

  // codes [8 q, 8 q + 8) of the thread's 32 in a register stage, to four
  // packed bf16 pairs (one quarter of what MOEQ_LSTORE writes)
  auto deq8 = [&](const u32x4* BR, int q, float SV, float CV, uint32_t* o4) {
    if constexpr (MX) {
      const uint32_t x = BR[0][q] & (SV != 0.f ? 0xFFFFFFFFu : 0u);
      o4[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, SV, 0));
      o4[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, SV, 1));
      o4[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, SV, 2));
      o4[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, SV, 3));
    } else {
      constexpr int kPer = 32 / BITS;
      constexpr uint32_t kMask = (1u << BITS) - 1u;
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const int ca = 8 * q + j, cb = ca + 1;
        const uint32_t xa = BR[(ca / kPer) / 4][(ca / kPer) % 4], xb = BR[(cb / kPer) / 4][(cb / kPer) % 4];
        o4[j / 2] = pack_bf16(fmaf(SV, (float)((xa >> (BITS * (ca % kPer))) & kMask), CV),
                              fmaf(SV, (float)((xb >> (BITS * (cb % kPer))) & kMask), CV));
      }
    }
  };
  // a step's MFMAs on LDS stage rbuf, with the next step (register stage
  // AR/BR, loaded one step earlier) dequantized and written to the other LDS
  // stage a quarter per 16-wide k slice, so the dequantization runs between
  // the MFMAs instead of after them (the other stage was last read before the
  // previous barrier)
  // MM false: a wave whose 128 rows all lie past the tile's last row (in an
  // expert's last, partial tile) only stages the next step, no MFMAs
  auto fused_step = [&](int rbuf, const u32x4* AR, const u32x4* BR, uint32_t SRAW, uint32_t CRAW, float MV,
                        auto MM) {
    const float SV = (MX ? e8m0_f32(SRAW) : bf16_to_f32(SRAW)) * MV;
    const float CV = (MX ? 0.f : bf16_to_f32(CRAW)) * MV;
    const uint16_t* As = gsm + rbuf * kStage;
    const uint16_t* Bs = As + kBM * kLds;
    uint16_t* Aw = gsm + (rbuf ^ 1) * kStage;
    u32x4* dB = reinterpret_cast<u32x4*>(&Aw[kBM * kLds + bc * kLds + bh * 32]);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int kof = kk * 16 + 8 * (lane >> 5);
      uint32_t o4[4];
      if constexpr (decltype(MM)::value) {
        bf16x8 af[4], bfr[2];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
          af[mi] = *reinterpret_cast<const bf16x8*>(&As[(wm * 128 + mi * 32 + (lane & 31)) * kLds + kof]);
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          bfr[ni] = *reinterpret_cast<const bf16x8*>(&Bs[(wn * 64 + ni * 32 + (lane & 31)) * kLds + kof]);
        deq8(BR, kk, SV, CV, o4);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ni], af[mi], acc[mi][ni], 0, 0, 0);
      } else {
        deq8(BR, kk, SV, CV, o4);
      }
      *reinterpret_cast<u32x4*>(&Aw[((tid >> 3) + 64 * kk) * kLds + aseg * 8]) = AR[kk];
      dB[kk] = u32x4{o4[0], o4[1], o4[2], o4[3]};
    }
  };

  // a step: the loads of step kt+2 go out first (into the register stage step
  // kt used), the MFMAs of step kt run on LDS stage kt % 2 while step kt+1
  // (loaded one step earlier) is written to the other LDS stage.  The body
  // has no branches (loads past the last step re-read it); both halves
  // always run their MFMAs, and with an odd step count the last half's B
  // stage is written with zero scale and bias so it adds nothing.
  const int klast = ksteps - 1;
  MOEQ_GLOAD(a0, b0, s0, c0, m0, 0);
  MOEQ_GLOAD(a1, b1, s1, c1, m1, min(1, klast));
  MOEQ_LSTORE(a0, b0, s0, c0, m0, 0);
  __syncthreads();
  auto kloop = [&](auto MM) {
    for (int kt = 0; kt < ksteps; kt += 2) {
      const float on = kt + 1 < ksteps ? 1.f : 0.f;
      MOEQ_GLOAD(a0, b0, s0, c0, m0, min(kt + 2, klast));
      if constexpr (!MX) {
        // affine: the loads go out before this step's MFMAs (the scheduler
        // would sink them), the next stage's dequantization between them
        __builtin_amdgcn_sched_barrier(0);
        fused_step(0, a1, b1, s1, c1, m1 * on, MM);
      } else {
        // mxfp4 (a few conversion instructions per stage): the MFMAs, then
        // the next stage; measured faster this way than interleaved
        if constexpr (decltype(MM)::value) mfma_step(0);
        MOEQ_LSTORE(a1, b1, s1, c1, m1 * on, 1);
      }
      __syncthreads();
      MOEQ_GLOAD(a1, b1, s1, c1, m1, min(kt + 3, klast));
      if constexpr (!MX) {
        __builtin_amdgcn_sched_barrier(0);
        fused_step(1, a0, b0, s0, c0, m0, MM);
      } else {
        if constexpr (decltype(MM)::value) mfma_step(1);
        MOEQ_LSTORE(a0, b0, s0, c0, m0, 0);
      }
      __syncthreads();
    }
  };
  // a wave whose rows all lie past the tile's count (the lower half of an
  // expert's last tile of at most 128 rows) skips its MFMAs: they would
  // multiply rows that are never stored
  if (wm * 128 < rows) kloop(std::true_type{});
  else kloop(std::false_type{});
#undef MOEQ_GLOAD
#undef MOEQ_LSTORE

  // ---- epilogue.  The transposed 32x32 accumulator: register r of lane l
  // holds output column 8*(r/4) + 4*(l/32) + r%4 of the tile's 32 and token
  // row l%32, so registers 4q..4q+3 are four consecutive columns of one row
  // and go out as one 8-byte (bf16) or 16-byte (fp32) store.
  auto pk4 = [](float a, float b, float c, float d) {
    return make_uint2(pack_bf16(a, b), pack_bf16(c, d));
  };
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int rl = wm * 128 + mi * 32 + (lane & 31);       // the lane's token row
    if (rl >= rows) continue;
    const int pair = s_pair[rl];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int cofs = 8 * q + 4 * (lane >> 5);             // first of the four columns
      if (MODE == 1) {
        const int i = nt * 128 + wn * 32 + cofs;
        if (i < N) {
          float hv[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) hv[u] = silu(acc[mi][0][4 * q + u]) * acc[mi][1][4 * q + u];
          uint16_t* o = reinterpret_cast<uint16_t*>(out) + (size_t)(row0 + rl) * N + i;
          if (i + 3 < N && (N & 3) == 0) {
            *reinterpret_cast<uint2*>(o) = pk4(hv[0], hv[1], hv[2], hv[3]);
          } else {
            for (int u = 0; u < 4 && i + u < N; ++u)
              o[u] = (uint16_t)(pack_bf16(hv[u], 0.f) & 0xFFFFu);
          }
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int n = nt * kBN + wn * 64 + ni * 32 + cofs;
          if (n >= N) continue;
          if (MODE == 2) {
            const float sw = s_w[rl];
            const float v0 = acc[mi][ni][4 * q] * sw, v1 = acc[mi][ni][4 * q + 1] * sw;
            const float v2 = acc[mi][ni][4 * q + 2] * sw, v3 = acc[mi][ni][4 * q + 3] * sw;
            uint16_t* o = reinterpret_cast<uint16_t*>(out) + (size_t)pair * N + n;
            if (n + 3 < N && (N & 3) == 0) {
              *reinterpret_cast<uint2*>(o) = pk4(v0, v1, v2, v3);
            } else {
              const float vv[4] = {v0, v1, v2, v3};
              for (int u = 0; u < 4 && n + u < N; ++u)
                o[u] = (uint16_t)(pack_bf16(vv[u], 0.f) & 0xFFFFu);
            }
          } else {
            float* o = reinterpret_cast<float*>(out) + (size_t)pair * N + n;
            if (n + 3 < N && (N & 3) == 0) {
              *reinterpret_cast<float4*>(o) = make_float4(acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1],
                                                          acc[mi][ni][4 * q + 2], acc[mi][ni][4 * q + 3]);
            } else {
              for (int u = 0; u < 4 && n + u < N; ++u) o[u] = acc[mi][ni][4 * q + u];
            }
          }
        }
      }
    }
  }
}

// y[t][c] = sum over slots k (in order) of ypair[t*K+k][c] (bf16 -> fp32); NaN
// for a pair whose expert index is out of range (its row was never computed).
__global__ void __launch_bounds__(256) k_combine(const uint16_t* __restrict__ ypair,
                                                 const int32_t* __restrict__ idx, int M, int K,
                                                 int H, int E, float* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // 8-column group
  const int64_t total = (int64_t)M * H / 8;
  if (i >= total) return;
  const int64_t t = (i * 8) / H;
  const int64_t c = i * 8 - t * H;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // the K rows' loads go out together (every pair row exists in the
  // workspace; an invalid pair's row is read and discarded), then the sums
  // in slot order
  constexpr int kB = 8;
  for (int k0 = 0; k0 < K; k0 += kB) {
    uint4 v[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j)
      if (k0 + j < K) v[j] = *reinterpret_cast<const uint4*>(ypair + (t * K + k0 + j) * H + c);
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      if (k0 + j >= K) break;
      const int e = idx[t * K + k0 + j];
      if (e >= 0 && e < E) {
        const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          s[2 * q] += bf16_to_f32(w[q] & 0xFFFFu);
          s[2 * q + 1] += bf16_to_f32(w[q] >> 16);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) s[q] = __builtin_nanf("");
      }
    }
  }
  float4* yo = reinterpret_cast<float4*>(y + t * H + c);
  yo[0] = make_float4(s[0], s[1], s[2], s[3]);
  yo[1] = make_float4(s[4], s[5], s[6], s[7]);
}

// rows whose expert index is out of range, and with `runs` (rows used in
// place: sorted indices) rows outside their expert's run, come out NaN
__global__ void __launch_bounds__(256) k_mark_invalid(const int32_t* __restrict__ idx, int n, int E,
                                                      int N, const int32_t* __restrict__ runs,
                                                      float* __restrict__ out) {
  const int row = blockIdx.x;
  const int e = idx[row];
  if (e >= 0 && e < E && (!runs || (runs[e] <= row && row < runs[e + 1]))) return;
  for (int c = threadIdx.x; c < N; c += blockDim.x) out[(size_t)row * N + c] = __builtin_nanf("");
}

template <int BITS, int MODE, bool MX = false>
static void gemm_launch(dim3 grid, hipStream_t s, const QT& W, const QT& W2, int N, int Kd,
                        const uint16_t* A, int a_div, const GatherWs& ws, const float* wts,
                        void* out, int ntn) {
  // two LDS stages of 147,456 bytes: above the default dynamic limit
  MOEQ_ALLOW_FULL_LDS((k_gqmm<BITS, MODE, MX>), kGemmLds);
  hipLaunchKernelGGL((k_gqmm<BITS, MODE, MX>), grid, dim3(kThreads), kGemmLds, s, W, W2, N, Kd, A,
                     a_div, ws, wts, out, ntn);
}

template <int MODE>
static void gemm_bits(int bits, dim3 grid, hipStream_t s, const QT& W, const QT& W2, int N, int Kd,
                      const uint16_t* A, int a_div, const GatherWs& ws, const float* wts,
                      void* out, int ntn) {
  if (W.mode == 1) gemm_launch<4, MODE, true>(grid, s, W, W2, N, Kd, A, a_div, ws, wts, out, ntn);
  else if (bits == 8) gemm_launch<8, MODE>(grid, s, W, W2, N, Kd, A, a_div, ws, wts, out, ntn);
  else if (bits == 4) gemm_launch<4, MODE>(grid, s, W, W2, N, Kd, A, a_div, ws, wts, out, ntn);
  else gemm_launch<2, MODE>(grid, s, W, W2, N, Kd, A, a_div, ws, wts, out, ntn);
}

static dim3 gemm_grid(const GatherWs& ws, int ntn) {
  const int items = ws.max_tiles * ntn;
  return dim3((unsigned)(((items + kXcd - 1) / kXcd) * kXcd));
}

int launch_gemm_gate_up(const QT& gate, const QT& up, const uint16_t* x, int K, const GatherWs& ws,
                        int n, hipStream_t s) {
  (void)n;
  const int I = gate.rows, H = gate.cols;
  const int ntn = (I + 127) / 128;
  gemm_bits<1>(gate.bits, gemm_grid(ws, ntn), s, gate, up, I, H, x, K, ws, nullptr, (void*)ws.h, ntn);
  return 0;
}

int launch_gemm_down(const QT& down, const float* w, const GatherWs& ws, int n, hipStream_t s) {
  (void)n;
  const int H = down.rows, I = down.cols;
  const int ntn = (H + kBN - 1) / kBN;
  gemm_bits<2>(down.bits, gemm_grid(ws, ntn), s, down, down, H, I, (const uint16_t*)ws.h, 1, ws, w,
               (void*)ws.ypair, ntn);
  return 0;
}

int launch_gemm_plain(const QT& W, const uint16_t* x, float* out, const GatherWs& ws, int n,
                      hipStream_t s) {
  (void)n;
  const int ntn = (W.rows + kBN - 1) / kBN;
  gemm_bits<0>(W.bits, gemm_grid(ws, ntn), s, W, W, W.rows, W.cols, x, 1, ws, nullptr, (void*)out, ntn);
  return 0;
}

int launch_mark_invalid_rows(const int32_t* idx, int n, int E, int N, const int32_t* runs, float* out,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_mark_invalid, dim3(n), dim3(256), 0, s, idx, n, E, N, runs, out);
  return 0;
}

int launch_combine(const uint16_t* ypair, const int32_t* idx, int M, int K, int H, int E, float* y,
                   hipStream_t s) {
  const int64_t total = (int64_t)M * H / 8;
  if (total == 0) return 0;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)blocks), dim3(256), 0, s, ypair, idx, M, K, H, E, y);
  return 0;
}

}  // namespace moeq
