// Decode expert forward (fp32 activations, any M): per selected expert the
// fused dequantize gate/up matvec with a SwiGLU epilogue, then the down
// projection with the weighted combine of all K experts (+ sigmoid-gated
// shared expert, + residual) for one output row inside one wave.
//
// Step order follows markbaseengine MOE_ROUTER_WORKS_BREAKTHROUGH ("Forward
// Pass Sequence": expertFusedGateUp, expertDown, accumulateResults) and the
// flash-moe-inference kernels swiglu and moe_combine_residual.  The down+
// combine wave adds the K expert terms in slot order, so the output does not
// depend on scheduling: no atomics, bitwise reproducible.
#include "common.h"
#include "launch.h"

namespace moeq {

// ---------------------------------------------------------------------------
// gate/up + SwiGLU: one wave per (token, slot, intermediate row).  Work items:
//   [0, M*K*I)              routed: h[t][k][i]
//   [M*K*I, +M*Is)          shared expert: hs[t][i]
//   [.., +M)                shared_expert_gate logit sg[t]
// ---------------------------------------------------------------------------
template <int BITS, int BITS_SH, int BITS_EG>
__global__ void __launch_bounds__(256) k_dec_gate_up(DecodeLayer L, const float* __restrict__ x,
                                                     const int32_t* __restrict__ idx, int M, int K,
                                                     float* __restrict__ ws) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t item = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  const int H = L.H, I = L.I, Is = L.Is;
  const int64_t n_routed = (int64_t)M * K * I;
  const int64_t n_shared = L.has_shared ? (int64_t)M * Is : 0;
  const int64_t n_eg = L.has_shared ? M : 0;
  if (item >= n_routed + n_shared + n_eg) return;

  float* h_routed = ws;
  float* h_shared = ws + n_routed;
  float* sg = h_shared + n_shared;

  if (item < n_routed + n_shared) {
    const bool routed = item < n_routed;
    int t, i;
    const uint32_t *qg, *qu;
    const uint16_t *sg_, *bg_, *su_, *bu_;
    float* out;
    bool valid = true;
    if (routed) {
      const int64_t p = item / I;  // pair = t*K + k
      i = (int)(item - p * I);
      t = (int)(p / K);
      const int e = idx[p];
      valid = e >= 0 && e < L.E;
      const int64_t row = (int64_t)(valid ? e : 0) * I + i;
      const int wpr = H / (32 / BITS);
      const int gpr = H / kGroup;
      qg = L.gate.q + row * wpr;
      qu = L.up.q + row * wpr;
      sg_ = L.gate.scales + row * gpr;
      bg_ = L.gate.biases + row * gpr;
      su_ = L.up.scales + row * gpr;
      bu_ = L.up.biases + row * gpr;
      out = h_routed + item;
    } else {
      const int64_t j = item - n_routed;
      t = (int)(j / Is);
      i = (int)(j - (int64_t)t * Is);
      const int wpr = H / (32 / BITS_SH);
      const int gpr = H / kGroup;
      qg = L.sh_gate.q + (int64_t)i * wpr;
      qu = L.sh_up.q + (int64_t)i * wpr;
      sg_ = L.sh_gate.scales + (int64_t)i * gpr;
      bg_ = L.sh_gate.biases + (int64_t)i * gpr;
      su_ = L.sh_up.scales + (int64_t)i * gpr;
      bu_ = L.sh_up.biases + (int64_t)i * gpr;
      out = h_shared + j;
    }
    const float* xt = x + (int64_t)t * H;
    float ag = 0.f, au = 0.f;
    if (routed) {
      constexpr int kCpc = 128 / BITS;
      const uint4* g4 = reinterpret_cast<const uint4*>(qg);
      const uint4* u4 = reinterpret_cast<const uint4*>(qu);
      for (int c = lane; c < H / kCpc; c += kWave) {
        const uint4 vg = g4[c], vu = u4[c];
        const int grp = (c * kCpc) / kGroup;
        const float s1 = bf16_to_f32(sg_[grp]), b1 = bf16_to_f32(bg_[grp]);
        const float s2 = bf16_to_f32(su_[grp]), b2 = bf16_to_f32(bu_[grp]);
        const float* xc = xt + c * kCpc;
#pragma unroll
        for (int j = 0; j < kCpc; j += 4) {
          const float4 xv = *reinterpret_cast<const float4*>(xc + j);
          const float xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            ag = fmaf(fmaf(s1, (float)chunk_code<BITS>(vg, j + u), b1), xs[u], ag);
            au = fmaf(fmaf(s2, (float)chunk_code<BITS>(vu, j + u), b2), xs[u], au);
          }
        }
      }
    } else {
      constexpr int kCpc = 128 / BITS_SH;
      const uint4* g4 = reinterpret_cast<const uint4*>(qg);
      const uint4* u4 = reinterpret_cast<const uint4*>(qu);
      for (int c = lane; c < H / kCpc; c += kWave) {
        const uint4 vg = g4[c], vu = u4[c];
        const int grp = (c * kCpc) / kGroup;
        const float s1 = bf16_to_f32(sg_[grp]), b1 = bf16_to_f32(bg_[grp]);
        const float s2 = bf16_to_f32(su_[grp]), b2 = bf16_to_f32(bu_[grp]);
        const float* xc = xt + c * kCpc;
#pragma unroll
        for (int j = 0; j < kCpc; j += 4) {
          const float4 xv = *reinterpret_cast<const float4*>(xc + j);
          const float xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            ag = fmaf(fmaf(s1, (float)chunk_code<BITS_SH>(vg, j + u), b1), xs[u], ag);
            au = fmaf(fmaf(s2, (float)chunk_code<BITS_SH>(vu, j + u), b2), xs[u], au);
          }
        }
      }
    }
    ag = wave_sum(ag);
    au = wave_sum(au);
    if (lane == 0) *out = valid ? silu(ag) * au : __builtin_nanf("");
  } else {
    // shared_expert_gate: one row of H
    const int t = (int)(item - n_routed - n_shared);
    constexpr int kCpc = 128 / BITS_EG;
    const uint4* q4 = reinterpret_cast<const uint4*>(L.sh_eg.q);
    const float* xt = x + (int64_t)t * H;
    float a = 0.f;
    for (int c = lane; c < H / kCpc; c += kWave) {
      const uint4 v = q4[c];
      const int grp = (c * kCpc) / kGroup;
      const float s = bf16_to_f32(L.sh_eg.scales[grp]), b = bf16_to_f32(L.sh_eg.biases[grp]);
      const float* xc = xt + c * kCpc;
#pragma unroll
      for (int j = 0; j < kCpc; j += 4) {
        const float4 xv = *reinterpret_cast<const float4*>(xc + j);
        a = fmaf(fmaf(s, (float)chunk_code<BITS_EG>(v, j + 0), b), xv.x, a);
        a = fmaf(fmaf(s, (float)chunk_code<BITS_EG>(v, j + 1), b), xv.y, a);
        a = fmaf(fmaf(s, (float)chunk_code<BITS_EG>(v, j + 2), b), xv.z, a);
        a = fmaf(fmaf(s, (float)chunk_code<BITS_EG>(v, j + 3), b), xv.w, a);
      }
    }
    a = wave_sum(a);
    if (lane == 0) sg[t] = a;
  }
}

// ---------------------------------------------------------------------------
// down + combine: a block stages token t's h (K*I + Is floats) in LDS and
// each wave produces whole output rows: y[t][r] = sum_k w_k (Wd_e_k[r] . h_k)
// + sigmoid(sg) (Wd_sh[r] . h_sh) + residual.  Lane-local terms are summed in
// slot order, then one fixed-order wave reduction.
// ---------------------------------------------------------------------------
constexpr int kDownRowsPerBlock = 16;

template <int BITS, int BITS_SH>
__global__ void __launch_bounds__(256) k_dec_down(DecodeLayer L, const int32_t* __restrict__ idx,
                                                  const float* __restrict__ wts, int M, int K,
                                                  const float* __restrict__ residual,
                                                  float* __restrict__ y,
                                                  const float* __restrict__ ws) {
  extern __shared__ float hs[];  // [K*I + Is]
  const int H = L.H, I = L.I, Is = L.Is;
  const int blocks_per_tok = (H + kDownRowsPerBlock - 1) / kDownRowsPerBlock;
  const int t = blockIdx.x / blocks_per_tok;
  const int r0 = (blockIdx.x - t * blocks_per_tok) * kDownRowsPerBlock;
  const int64_t n_routed = (int64_t)M * K * I;
  const int nh = K * I + (L.has_shared ? Is : 0);
  const float* ht = ws + (int64_t)t * K * I;
  for (int j = threadIdx.x; j < K * I; j += blockDim.x) hs[j] = ht[j];
  if (L.has_shared) {
    const float* hsh = ws + n_routed + (int64_t)t * Is;
    for (int j = threadIdx.x; j < Is; j += blockDim.x) hs[K * I + j] = hsh[j];
  }
  __syncthreads();
  (void)nh;

  float gate_scale = 0.f;
  if (L.has_shared) {
    const float sgv = ws[n_routed + (int64_t)M * Is + t];
    gate_scale = 1.0f / (1.0f + __expf(-sgv));
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  constexpr int kCpc = 128 / BITS;
  constexpr int kCpcS = 128 / BITS_SH;
  const int ch = I / kCpc;                       // chunks per routed down row
  const int chs = L.has_shared ? Is / kCpcS : 0; // chunks of the shared down row
  const int total = K * ch + chs;
  for (int rr = wid; rr < kDownRowsPerBlock; rr += blockDim.x / kWave) {
    const int r = r0 + rr;
    if (r >= H) break;
    float acc = 0.f;
    for (int c = lane; c < total; c += kWave) {
      if (c < K * ch) {
        const int k = c / ch;
        const int cc = c - k * ch;
        const int e = idx[(int64_t)t * K + k];
        const bool valid = e >= 0 && e < L.E;
        const int64_t row = (int64_t)(valid ? e : 0) * H + r;
        const uint4 v = reinterpret_cast<const uint4*>(L.down.q + row * (I / (32 / BITS)))[cc];
        const int grp = (cc * kCpc) / kGroup;
        const float s = bf16_to_f32(L.down.scales[row * (I / kGroup) + grp]);
        const float b = bf16_to_f32(L.down.biases[row * (I / kGroup) + grp]);
        const float* hk = hs + k * I + cc * kCpc;
        float d = 0.f;
#pragma unroll
        for (int j = 0; j < kCpc; ++j) d = fmaf(fmaf(s, (float)chunk_code<BITS>(v, j), b), hk[j], d);
        acc = fmaf(valid ? wts[(int64_t)t * K + k] : __builtin_nanf(""), d, acc);
      } else {
        const int cc = c - K * ch;
        const uint4 v = reinterpret_cast<const uint4*>(L.sh_down.q + (int64_t)r * (Is / (32 / BITS_SH)))[cc];
        const int grp = (cc * kCpcS) / kGroup;
        const float s = bf16_to_f32(L.sh_down.scales[(int64_t)r * (Is / kGroup) + grp]);
        const float b = bf16_to_f32(L.sh_down.biases[(int64_t)r * (Is / kGroup) + grp]);
        const float* hk = hs + K * I + cc * kCpcS;
        float d = 0.f;
#pragma unroll
        for (int j = 0; j < kCpcS; ++j) d = fmaf(fmaf(s, (float)chunk_code<BITS_SH>(v, j), b), hk[j], d);
        acc = fmaf(gate_scale, d, acc);
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) {
      if (residual) acc += residual[(int64_t)t * H + r];
      y[(int64_t)t * H + r] = acc;
    }
  }
}

size_t decode_lds_bytes(const DecodeLayer& L, int K) {
  return sizeof(float) * ((size_t)K * L.I + (L.has_shared ? L.Is : 0));
}

template <int B, int BS, int BE>
static void run_decode(const DecodeLayer& L, const float* x, const int32_t* idx, const float* w,
                       int M, int K, const float* residual, float* y, float* ws, hipStream_t s) {
  const int64_t items = (int64_t)M * K * L.I + (L.has_shared ? (int64_t)M * L.Is + M : 0);
  const int64_t blocks = (items + 3) / 4;
  hipLaunchKernelGGL((k_dec_gate_up<B, BS, BE>), dim3((unsigned)blocks), dim3(256), 0, s, L, x,
                     idx, M, K, ws);
  const int bpt = (L.H + kDownRowsPerBlock - 1) / kDownRowsPerBlock;
  hipLaunchKernelGGL((k_dec_down<B, BS>), dim3((unsigned)(M * bpt)), dim3(256),
                     decode_lds_bytes(L, K), s, L, idx, w, M, K, residual, y, ws);
}

int launch_decode_forward(const DecodeLayer& L, const float* x, const int32_t* idx, const float* w,
                          int M, int K, const float* residual, float* y, float* ws, hipStream_t s) {
  const int b = L.gate.bits;
  const int bs = L.has_shared ? L.sh_gate.bits : b;
  const int be = L.has_shared ? L.sh_eg.bits : 8;
  // expert bits x shared-expert bits x shared-gate bits
#define MOEQ_DEC(B_, BS_, BE_)                                                     \
  if (b == B_ && bs == BS_ && be == BE_) {                                        \
    run_decode<B_, BS_, BE_>(L, x, idx, w, M, K, residual, y, ws, s);             \
    return 0;                                                                     \
  }
#define MOEQ_DEC_BE(B_, BS_) MOEQ_DEC(B_, BS_, 8) MOEQ_DEC(B_, BS_, 4) MOEQ_DEC(B_, BS_, 2)
#define MOEQ_DEC_BS(B_) MOEQ_DEC_BE(B_, 8) MOEQ_DEC_BE(B_, 4) MOEQ_DEC_BE(B_, 2)
  MOEQ_DEC_BS(8)
  MOEQ_DEC_BS(4)
  MOEQ_DEC_BS(2)
#undef MOEQ_DEC_BS
#undef MOEQ_DEC_BE
#undef MOEQ_DEC
  return -9;
}

}  // namespace moeq
