// Router GEMM + score + wavefront top-k + gate weights, fused in one kernel.
//
// Page "MoE sparse activation: principles and engineering practice"
// (kapook.pages.dev), s3.1 Router: a bias-free linear map d -> E, the top-k of
// the logits, sorted, and softmax over the chosen logits as gate weights.
// Page "GPT-4 has 1.8T parameters but uses 2% per token" (mlqm.cn), s3.1:
// Gumbel noise -log(-log u) added to the logits and a temperature (0.5)
// before the softmax.  Page "From sparse MoE to conditional memory"
// (m.nxbn.cn), gating-network implementation: a per-expert bias added to the
// scores before the top-k.  Sigmoid scores normalised over the chosen experts
// (bias for selection only) are the fine-grained workload's rule.
//
// One block = BT tokens x all experts.  Phase 1 computes z[BT][E] with f32 FMAs
// from LDS tiles (K split across the four waves, blocked partial sums so the
// error stays ~1e-7 of |z| at K = 12800).  Phase 2 gives each wave one token at
// a time: lane l holds experts l, l+64, ... in registers, computes the keys in
// float32 in a fixed operation order, and runs k rounds of a wave arg-max with
// ties to the lower expert index.  Gate weights are formed in float64 and
// rounded once.
#include <float.h>

#include "common.h"

namespace moe {
namespace {

struct Cand {
  float key;
  float basis;
  int e;  // INT32_MAX = no candidate
};

__device__ __forceinline__ bool better(const Cand& a, const Cand& b) {
  if (a.e == INT32_MAX) return false;
  if (b.e == INT32_MAX) return true;
  return a.key > b.key || (a.key == b.key && a.e < b.e);
}

__device__ __forceinline__ Cand wave_argmax(Cand c) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    Cand o;
    o.key = __shfl_xor(c.key, m);
    o.basis = __shfl_xor(c.basis, m);
    o.e = __shfl_xor(c.e, m);
    if (better(o, c)) c = o;
  }
  return c;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

template <bool BF16X, int EMAX, int BT, int ESPLIT, int TM, int TN>
__global__ __launch_bounds__(256) void route_kernel(RouteLaunch a) {
  constexpr int KSPLIT = 4 / ESPLIT;
  constexpr int KW = 32;             // k per wave per tile
  constexpr int KT = KSPLIT * KW;    // k per tile
  constexpr int EW = EMAX / ESPLIT;  // experts per wave
  constexpr int EG = EW / TN;        // expert groups per wave
  constexpr int TG = BT / TM;        // token groups per wave
  constexpr int EPL = (EMAX + 63) / 64;
  static_assert(EG * TG == 64, "one wave covers the tile");

  __shared__ float xs[BT][KT + 1];
  __shared__ __attribute__((aligned(16))) float wsm[KT][EMAX];
  __shared__ float zs[KSPLIT][BT][EMAX];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ksub = wave % KSPLIT;
  const int esub = wave / KSPLIT;
  const int tg = lane / EG;
  const int eg = lane % EG;
  const int t0 = blockIdx.x * BT;
  const int T = a.T, d = a.d, E = a.E;

  float acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = 0.f;

  for (int k0 = 0; k0 < d; k0 += KT) {
    // ---- stage x[BT][KT] (as f32) and W_r[KT][EMAX] (zero past E)
    if (BF16X) {
      const uint16_t* x = (const uint16_t*)a.x;
      constexpr int CH = BT * KT / 8;
      for (int c = tid; c < CH; c += 256) {
        int r = c / (KT / 8), c8 = c % (KT / 8);
        int t = t0 + r;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (t < T) v = *(const uint4*)(x + (size_t)t * d + k0 + c8 * 8);
        float* dst = &xs[r][c8 * 8];
        dst[0] = bf16_bits_to_f32(v.x & 0xffff); dst[1] = bf16_bits_to_f32(v.x >> 16);
        dst[2] = bf16_bits_to_f32(v.y & 0xffff); dst[3] = bf16_bits_to_f32(v.y >> 16);
        dst[4] = bf16_bits_to_f32(v.z & 0xffff); dst[5] = bf16_bits_to_f32(v.z >> 16);
        dst[6] = bf16_bits_to_f32(v.w & 0xffff); dst[7] = bf16_bits_to_f32(v.w >> 16);
      }
    } else {
      const float* x = (const float*)a.x;
      constexpr int CH = BT * KT / 4;
      for (int c = tid; c < CH; c += 256) {
        int r = c / (KT / 4), c4 = c % (KT / 4);
        int t = t0 + r;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t < T) v = *(const float4*)(x + (size_t)t * d + k0 + c4 * 4);
        float* dst = &xs[r][c4 * 4];
        dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
      }
    }
    for (int c = tid; c < KT * EMAX; c += 256) {
      int r = c / EMAX, e = c % EMAX;
      wsm[r][e] = (e < E) ? a.w_router[(size_t)(k0 + r) * E + e] : 0.f;
    }
    __syncthreads();

    float part[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) part[i][j] = 0.f;
    const int kb = ksub * KW;
    const int eb = esub * EW + eg * TN;
#pragma unroll 4
    for (int kk = 0; kk < KW; ++kk) {
      float xv[TM], wv[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) xv[i] = xs[tg * TM + i][kb + kk];
#pragma unroll
      for (int j = 0; j < TN; ++j) wv[j] = wsm[kb + kk][eb + j];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) part[i][j] = fmaf(xv[i], wv[j], part[i][j]);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] += part[i][j];
    __syncthreads();
  }

  // ---- combine the K-split partial sums in a fixed order
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) zs[ksub][tg * TM + i][esub * EW + eg * TN + j] = acc[i][j];
  __syncthreads();
  if (KSPLIT > 1) {
    for (int c = tid; c < BT * EMAX; c += 256) {
      int r = c / EMAX, e = c % EMAX;
      float z = zs[0][r][e];
#pragma unroll
      for (int s = 1; s < KSPLIT; ++s) z += zs[s][r][e];
      zs[0][r][e] = z;
    }
    __syncthreads();
  }

  // ---- keys, wavefront top-k, gate weights: one token per wave at a time
  const float tau = a.tau;
  for (int tl = wave; tl < BT; tl += 4) {
    const int t = t0 + tl;
    if (t >= T) break;  // uniform across the wave; no barrier below
    float key[EPL], basis[EPL];
    bool taken[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      taken[i] = !(e < E);
      key[i] = 0.f;
      basis[i] = 0.f;
      if (e < E) {
        const float z = zs[0][tl][e];
        if (a.logits) a.logits[(size_t)t * E + e] = z;
        if (a.score == MOE_SCORE_SOFTMAX) {
          float l = z;
          if (a.bias_mode == MOE_BIAS_LOGIT) l = l + a.bias[e];
          if (a.gumbel_u) {
            const double u = (double)a.gumbel_u[(size_t)t * E + e];
            l = l + (float)(-log(-log(u)));
          }
          l = l / tau;
          basis[i] = l;
          key[i] = (a.bias_mode == MOE_BIAS_SELECT_ONLY) ? l + a.bias[e] : l;
        } else {
          const float s = (float)(1.0 / (1.0 + exp(-(double)z)));
          basis[i] = s;
          key[i] = (a.bias_mode == MOE_BIAS_SELECT_ONLY) ? s + a.bias[e] : s;
        }
      }
    }

    // k rounds of arg-max; slot j of the result is owned by lane j % 64, register j / 64
    int sel_e[4];
    float sel_b[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) { sel_e[s] = 0; sel_b[s] = 0.f; }
    for (int j = 0; j < a.k; ++j) {
      Cand c{-FLT_MAX, 0.f, INT32_MAX};
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        Cand o{key[i], basis[i], taken[i] ? INT32_MAX : lane + 64 * i};
        if (better(o, c)) c = o;
      }
      c = wave_argmax(c);
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (c.e == lane + 64 * i) taken[i] = true;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if ((j >> 6) == s && (j & 63) == lane) { sel_e[s] = c.e; sel_b[s] = c.basis; }
    }

    // gate weights in float64
    double w[4] = {0.0, 0.0, 0.0, 0.0};
    if (a.score == MOE_SCORE_SOFTMAX) {
      if (a.renormalize) {
        float m = -FLT_MAX;
#pragma unroll
        for (int s = 0; s < 4; ++s)
          if (lane + 64 * s < a.k) m = fmaxf(m, sel_b[s]);
        m = wave_max(m);
        double part = 0.0;
#pragma unroll
        for (int s = 0; s < 4; ++s)
          if (lane + 64 * s < a.k) { w[s] = exp((double)sel_b[s] - (double)m); part += w[s]; }
        const double sum = wave_sum(part);
#pragma unroll
        for (int s = 0; s < 4; ++s) w[s] /= sum;
      } else {
        float M = -FLT_MAX;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (lane + 64 * i < E) M = fmaxf(M, basis[i]);
        M = wave_max(M);
        double part = 0.0;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (lane + 64 * i < E) part += exp((double)basis[i] - (double)M);
        const double sum = wave_sum(part);
#pragma unroll
        for (int s = 0; s < 4; ++s)
          if (lane + 64 * s < a.k) w[s] = exp((double)sel_b[s] - (double)M) / sum;
      }
    } else {
      double part = 0.0;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (lane + 64 * s < a.k) { w[s] = (double)sel_b[s]; part += w[s]; }
      if (a.renormalize) {
        const double sum = wave_sum(part);
#pragma unroll
        for (int s = 0; s < 4; ++s) w[s] /= sum;
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int j = lane + 64 * s;
      if (j < a.k) {
        a.topk_idx[(size_t)t * a.k + j] = sel_e[s];
        a.topk_w[(size_t)t * a.k + j] = (float)w[s];
      }
    }
  }
}

template <bool BF16X, int EMAX, int BT, int ESPLIT, int TM, int TN>
moe_status launch_one(const RouteLaunch& a, hipStream_t s) {
  const int grid = (int)ceil_div(a.T, BT);
  int tok = begin_launch("route_topk", s);
  hipLaunchKernelGGL((route_kernel<BF16X, EMAX, BT, ESPLIT, TM, TN>), dim3(grid), dim3(256), 0, s, a);
  return end_launch(tok, s);
}

template <bool BF16X>
moe_status dispatch(const RouteLaunch& a, hipStream_t s) {
  if (a.E <= 8) return launch_one<BF16X, 8, 16, 1, 2, 1>(a, s);
  if (a.E <= 16) return launch_one<BF16X, 16, 16, 1, 2, 2>(a, s);
  if (a.E <= 32) return launch_one<BF16X, 32, 32, 1, 4, 4>(a, s);
  if (a.E <= 64) return launch_one<BF16X, 64, 32, 1, 4, 8>(a, s);
  if (a.E <= 128) return launch_one<BF16X, 128, 32, 2, 4, 8>(a, s);
  return launch_one<BF16X, 256, 32, 4, 4, 8>(a, s);
}

}  // namespace

moe_status launch_route(const RouteLaunch& a, hipStream_t s) {
  if (a.T == 0) return MOE_OK;
  return a.act_dtype == MOE_BF16 ? dispatch<true>(a, s) : dispatch<false>(a, s);
}

}  // namespace moe
