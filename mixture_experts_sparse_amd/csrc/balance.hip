// Load-balancing statistics of a routed batch and the loss-free bias step.
//
// Page "MoE sparse activation: principles and engineering practice"
// (kapook.pages.dev), s4.3 training stability: the auxiliary loss is the sum
// over experts of the mean router probability times the number of times the
// expert was chosen.  Router probability of (t, e): the distribution the gate
// weights are drawn from before the top-k -- the softmax over all experts of
// the weight basis for softmax scoring, the sigmoid scores normalised to sum 1
// for sigmoid scoring (the selection-only bias is not part of either).
//
// Page "From sparse MoE to conditional memory" (m.nxbn.cn), gating network
// code: without an auxiliary loss, each step sets
//     bias <- decay * bias - rate * load / (mean(load) + 1e-8)
// with load = how often each expert was chosen over all top-k slots.
//
// Everything is reduced in a fixed order in float64 (per lane, a fixed wave
// butterfly, the block's waves in index order, then each expert's block
// partials by strided sums meeting in a fixed tree), so the results do not
// depend on scheduling; values are rounded to float32 once at the end.
#include <float.h>

#include "common.h"
#include "route_keys.h"

namespace moe {
namespace {

constexpr int kTokPerBlock = 16;  // 4 tokens per wave

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

struct StatsParams {
  const float* logits;
  const float* bias;
  const float* gumbel_u;
  double* part;  // [E][blocks]: per-block sums of the probabilities
  int blocks;
  int T, E, score, bias_mode;
  float tau;
};

// Sum of each expert's router probability over the block's tokens; one wave
// per token, lane l holds experts l, l + 64, ...
template <int EPL>
__global__ __launch_bounds__(256) void stats_kernel(StatsParams p) {
  __shared__ double red[4][64 * EPL];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int E = p.E;
  double acc[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) acc[i] = 0.0;
  const int t_end = min(p.T, (int)(blockIdx.x + 1) * kTokPerBlock);
  for (int t = blockIdx.x * kTokPerBlock + w; t < t_end; t += 4) {
    float b[EPL];
    bool ok[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      ok[i] = e < E;
      b[i] = 0.f;
      if (ok[i]) {
        const size_t te = (size_t)t * E + e;
        b[i] = key_basis(p.logits[te], e, te, p.score, p.bias_mode, p.bias, p.gumbel_u, p.tau).basis;
      }
    }
    if (p.score == MOE_SCORE_SOFTMAX) {
      float m = -FLT_MAX;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (ok[i]) m = fmaxf(m, b[i]);
      m = wave_max_f(m);
      double ex[EPL], s = 0.0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        ex[i] = ok[i] ? exp((double)b[i] - (double)m) : 0.0;
        s += ex[i];
      }
      s = wave_sum_d(s);
#pragma unroll
      for (int i = 0; i < EPL; ++i) acc[i] += ex[i] / s;
    } else {
      double s = 0.0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) s += ok[i] ? (double)b[i] : 0.0;
      s = wave_sum_d(s);
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (ok[i]) acc[i] += (double)b[i] / s;
    }
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) red[w][lane + 64 * i] = acc[i];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    p.part[(size_t)e * p.blocks + blockIdx.x] = ((red[0][e] + red[1][e]) + red[2][e]) + red[3][e];
}

// Block e: prob_mean[e] = (sum of expert e's block partials) / T.  Thread i adds
// blocks i, i + 256, ... in order; the 256 sums then meet in a fixed tree.
__global__ __launch_bounds__(256) void stats_finish_kernel(const double* __restrict__ part, int blocks, int T,
                                                           float* __restrict__ prob_mean,
                                                           double* __restrict__ pm_exact) {
  __shared__ double red[256];
  const int e = blockIdx.x, tid = threadIdx.x;
  double s = 0.0;
  for (int b = tid; b < blocks; b += 256) s += part[(size_t)e * blocks + b];
  red[tid] = s;
  __syncthreads();
  for (int h = 128; h >= 1; h >>= 1) {
    if (tid < h) red[tid] += red[tid + h];
    __syncthreads();
  }
  if (tid == 0) {
    const double P = T > 0 ? red[0] / (double)T : 0.0;
    prob_mean[e] = (float)P;
    pm_exact[e] = P;
  }
}

// aux = sum_e prob_mean[e] * counts[e], in expert order (from the unrounded means)
__global__ __launch_bounds__(256) void stats_aux_kernel(const double* __restrict__ pm_exact,
                                                        const int32_t* __restrict__ counts, int E,
                                                        float* __restrict__ aux) {
  __shared__ double terms[256];
  if ((int)threadIdx.x < E) terms[threadIdx.x] = pm_exact[threadIdx.x] * (double)counts[threadIdx.x];
  __syncthreads();
  if (threadIdx.x == 0) {
    double a = 0.0;
    for (int e = 0; e < E; ++e) a += terms[e];
    aux[0] = (float)a;
  }
}

// bias[e] <- decay * bias[e] - rate * counts[e] / (mean(counts) + 1e-8), in float64
__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ counts, float* __restrict__ bias,
                                                          int E, float decay, float rate) {
  __shared__ double c[256];
  __shared__ double mean;
  if ((int)threadIdx.x < E) c[threadIdx.x] = (double)counts[threadIdx.x];
  __syncthreads();
  if (threadIdx.x == 0) {
    double s = 0.0;  // integer counts: the sum is exact in any order
    for (int e = 0; e < E; ++e) s += c[e];
    mean = s / (double)E;
  }
  __syncthreads();
  if ((int)threadIdx.x < E) {
    const double ratio = c[threadIdx.x] / (mean + 1e-8);
    bias[threadIdx.x] = (float)((double)decay * (double)bias[threadIdx.x] - (double)rate * ratio);
  }
}

}  // namespace

int64_t router_stats_ws_bytes(int T, int E) {
  // per-block partials [E][blocks], then the unrounded means [E]
  return ((int64_t)ceil_div(std::max(T, 1), kTokPerBlock) + 1) * E * (int64_t)sizeof(double);
}

moe_status launch_router_stats(const RouterStatsLaunch& a, hipStream_t s) {
  const int blocks = a.T > 0 ? (int)ceil_div(a.T, kTokPerBlock) : 0;
  double* pm_exact = a.part + (size_t)std::max(blocks, 1) * a.E;
  StatsParams p{a.logits, a.bias, a.gumbel_u, a.part, blocks, a.T, a.E, a.score, a.bias_mode, a.tau};
  int tok = begin_launch("balance_stats", s);
  if (blocks > 0) {
    if (a.E <= 64) hipLaunchKernelGGL(stats_kernel<1>, dim3(blocks), dim3(256), 0, s, p);
    else if (a.E <= 128) hipLaunchKernelGGL(stats_kernel<2>, dim3(blocks), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(stats_kernel<4>, dim3(blocks), dim3(256), 0, s, p);
  }
  moe_status st = end_launch(tok, s);
  if (st != MOE_OK) return st;
  tok = begin_launch("balance_finish", s);
  hipLaunchKernelGGL(stats_finish_kernel, dim3(a.E), dim3(256), 0, s, a.part, blocks, a.T, a.prob_mean, pm_exact);
  if (a.aux) hipLaunchKernelGGL(stats_aux_kernel, dim3(1), dim3(256), 0, s, pm_exact, a.counts, a.E, a.aux);
  return end_launch(tok, s);
}

moe_status launch_bias_update(const int32_t* counts, float* bias, int E, float decay, float rate, hipStream_t s) {
  int tok = begin_launch("bias_update", s);
  hipLaunchKernelGGL(bias_update_kernel, dim3(1), dim3(256), 0, s, counts, bias, E, decay, rate);
  return end_launch(tok, s);
}

}  // namespace moe
