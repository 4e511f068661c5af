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
// bf16 activations (the MFMA path):
//   router_prep   W_r [d,E] f32 -> Wt [3][EP][d] bf16 with W = hi + mid + lo
//                 exactly (each part the bf16 rounding of what the previous
//                 parts leave), transposed so K is contiguous for the MFMA
//   router_mfma   z partials over d-slices: x (bf16, exact) times hi, mid and
//                 lo on v_mfma_f32_16x16x32_bf16, accumulated in f32 -- every
//                 product is exact, so z matches an f32 router to ~1e-7 at a
//                 third of the bf16 MFMA rate; 8 waves x 32 tokens per block,
//                 W tiles shared through LDS, d split across blocks so all CUs
//                 work, partials written in [split][T][EP]
//   topk          one wave per token: z = partials summed in split order, then
//                 the keys / top-k / weights below
// f32 activations (tiny workloads): one fused SIMT kernel -- phase 1 computes
// z[BT][E] with f32 FMAs from LDS tiles (K split across the four waves,
// blocked partial sums), phase 2 is the same per-token routine.
//
// Per-token routine: lane l holds experts l, l+64, ... in registers, computes
// the keys in float32 in a fixed operation order, and runs k rounds of a wave
// arg-max with ties to the lower expert index.  Gate weights are formed in
// float64 and rounded once.
#include <float.h>

#include <algorithm>
#include <atomic>

#include "common.h"
#include "route_keys.h"

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

// Keys, wavefront top-k and gate weights of token t, executed by one whole wave.
// zget(e) returns the token's f32 logit of expert e (e < E).  Lane l holds
// experts l, l + 64, ... in registers; k rounds of a wave arg-max pick the
// largest keys, ties to the lower index; weights are formed in float64.
template <int EPL, typename ZGet>
__device__ __forceinline__ void route_token(const RouteLaunch& a, int t, int lane, ZGet zget) {
  const int E = a.E;
  const float tau = a.tau;
  float key[EPL], basis[EPL];
  bool taken[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    taken[i] = !(e < E);
    key[i] = 0.f;
    basis[i] = 0.f;
    if (e < E) {
      const float z = zget(e);
      if (a.logits) a.logits[(size_t)t * E + e] = z;
      const KeyBasis kb = key_basis(z, e, (size_t)t * E + e, a.score, a.bias_mode, a.bias, a.gumbel_u, tau);
      basis[i] = kb.basis;
      key[i] = kb.key;
    }
  }

  // k rounds of arg-max; slot j of the result is owned by lane j % 64, register j / 64
  int sel_e[4];
  float sel_b[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) { sel_e[s] = 0; sel_b[s] = 0.f; }
  // group-limited routing: topk_groups rounds of the same arg-max pick the
  // groups (a group's score is its largest key, so the best remaining expert
  // names the best remaining group); every expert outside them is then taken
  if (a.n_groups > 1) {
    const int gsz = E / a.n_groups;
    bool gone[EPL], kept[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      gone[i] = taken[i];
      kept[i] = false;
    }
    for (int g = 0; g < a.topk_groups; ++g) {
      Cand c{-FLT_MAX, 0.f, INT32_MAX};
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        Cand o{key[i], basis[i], gone[i] ? INT32_MAX : lane + 64 * i};
        if (better(o, c)) c = o;
      }
      c = wave_argmax(c);
      const int grp = c.e / gsz;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (!taken[i] && (lane + 64 * i) / gsz == grp) {
          gone[i] = true;
          kept[i] = true;
        }
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) taken[i] = taken[i] || !kept[i];
  }

  // k + fb rounds: the top-k, then the fallback experts for overflow re-routing
  for (int j = 0; j < a.k + a.fb; ++j) {
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
    if (j < a.k + a.fb) a.topk_idx[(size_t)t * (a.k + a.fb) + j] = sel_e[s];
    if (j < a.k) a.topk_w[(size_t)t * a.k + j] = (float)w[s];
  }
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
  for (int tl = wave; tl < BT; tl += 4) {
    const int t = t0 + tl;
    if (t >= T) break;  // uniform across the wave; no barrier below
    route_token<EPL>(a, t, lane, [&](int e) { return zs[0][tl][e]; });
  }
}

// ---------------------------------------------------------------- MFMA path
#define MOE_GPTR(p) ((const __attribute__((address_space(1))) void*)(p))
#define MOE_LPTR(p) ((__attribute__((address_space(3))) void*)(p))

// LDS a one-token-block router may hold its whole split d-slice in (dynamic LDS)
constexpr size_t kFusedRouterLds = 96 * 1024;

// s_waitcnt immediate (gfx9 encoding): vmcnt(n) alone
constexpr unsigned vmcnt_imm_r(int n) { return 0x0F70u | (unsigned)(n & 15) | ((unsigned)(n >> 4) << 14); }

__device__ __forceinline__ void bar() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// W_r [d][E] f32 -> Wt [3][EP][d] bf16 (rows e >= E are zero).  Block: 32 k x
// 64 e, one 8-wide k chunk of one expert per thread; the tile's eight loads per
// thread are all requested before any is used.
__global__ __launch_bounds__(256) void router_prep_kernel(const float* __restrict__ w, uint16_t* __restrict__ wt,
                                                          int d, int E, int EP) {
  __shared__ float tile[32][65];
  const int k0 = blockIdx.x * 32, e0 = blockIdx.y * 64;
  float v8[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int i = threadIdx.x + u * 256;
    const int r = i / 64, c = i % 64;
    v8[u] = (e0 + c < E) ? w[(size_t)(k0 + r) * E + e0 + c] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int i = threadIdx.x + u * 256;
    tile[i / 64][i % 64] = v8[u];
  }
  __syncthreads();
  const int el = threadIdx.x / 4, kc = threadIdx.x % 4;  // expert, 8-wide k chunk
  const int e = e0 + el;
  if (e >= EP) return;
  uint32_t hi[4], mid[4], lo[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t h2 = 0, m2 = 0, l2 = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float v = tile[kc * 8 + q * 2 + h][el];
      const uint16_t bh = f32_to_bf16_rne(v);
      const float r1 = v - bf16_bits_to_f32(bh);
      const uint16_t bm = f32_to_bf16_rne(r1);
      const float r2 = r1 - bf16_bits_to_f32(bm);
      const uint16_t bl = f32_to_bf16_rne(r2);
      h2 |= (uint32_t)bh << (16 * h);
      m2 |= (uint32_t)bm << (16 * h);
      l2 |= (uint32_t)bl << (16 * h);
    }
    hi[q] = h2; mid[q] = m2; lo[q] = l2;
  }
  const size_t o = (size_t)e * d + k0 + kc * 8;
  *(uint4*)(wt + o) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  *(uint4*)(wt + (size_t)EP * d + o) = make_uint4(mid[0], mid[1], mid[2], mid[3]);
  *(uint4*)(wt + (size_t)2 * EP * d + o) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
}

struct RouterParams {
  const uint16_t* x;   // [T, d]
  const uint16_t* wt;  // [3][EP][d]
  float* part;         // [split][T][EP]
  int T, d, kslice;
};

// z partial of 256 tokens x EP experts over one d-slice (blockIdx.y).  8 waves,
// wave w owns tokens 32 w .. 32 w + 31 and every expert.
template <int EP>
__global__ __launch_bounds__(512, 1) void router_mfma_kernel(RouterParams p) {
  constexpr int NF = EP / 16;
  constexpr int ROWS = 3 * EP;          // B rows: split-major (hi, mid, lo)
  constexpr int STAGE = ROWS * 64;      // 32 k (64 bytes) per row
  constexpr int NINS = ROWS / 16;       // 16-row load instructions per stage
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = p.T, d = p.d;
  const int t0 = blockIdx.x * 256;
  const int kb = blockIdx.y * p.kslice, ksteps = p.kslice / 32;
  const int kg = lane >> 4;
  // A fragments straight from global memory (rows past T repeat the last row)
  const uint16_t* xa0 = p.x + (size_t)min(t0 + w * 32 + (lane & 15), T - 1) * d + kb + kg * 8;
  const uint16_t* xa1 = p.x + (size_t)min(t0 + w * 32 + 16 + (lane & 15), T - 1) * d + kb + kg * 8;
  // B tile loads: 16 rows x 64 bytes per instruction, 16-byte chunk c of row r at slot c ^ ((r >> 1) & 3)
  const int dr = lane >> 2;
  const int dc = (lane & 3) ^ ((dr >> 1) & 3);
  const uint16_t* wsrc = p.wt + (size_t)dr * d + kb + dc * 8;
  const uint32_t bfrag = (uint32_t)((lane & 15) * 64 + ((kg ^ (((lane & 15) >> 1) & 3)) * 16));
  auto issue = [&](int ks) {
    uint8_t* st = smem + (ks & 1) * STAGE;
    for (int q = w; q < NINS; q += 8)
      __builtin_amdgcn_global_load_lds(MOE_GPTR(wsrc + (size_t)q * 16 * d + ks * 32), MOE_LPTR(st + q * 1024),
                                       16, 0, 0);
  };
  f32x4_t acc[2][NF];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < NF; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  issue(0);
  bf16x8_t a0 = *(const bf16x8_t*)xa0, a1 = *(const bf16x8_t*)xa1;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  bar();
  for (int ks = 0; ks < ksteps; ++ks) {
    bf16x8_t n0 = a0, n1 = a1;
    if (ks + 1 < ksteps) {
      issue(ks + 1);
      n0 = *(const bf16x8_t*)(xa0 + (ks + 1) * 32);
      n1 = *(const bf16x8_t*)(xa1 + (ks + 1) * 32);
    }
    const uint8_t* st = smem + (ks & 1) * STAGE;
#pragma unroll
    for (int n = 0; n < NF; ++n) {
      const bf16x8_t bh = *(const bf16x8_t*)(st + bfrag + (n * 16) * 64);
      const bf16x8_t bm = *(const bf16x8_t*)(st + bfrag + (EP + n * 16) * 64);
      const bf16x8_t bl = *(const bf16x8_t*)(st + bfrag + (2 * EP + n * 16) * 64);
      acc[0][n] = mfma16x16x32(a0, bh, acc[0][n]);
      acc[1][n] = mfma16x16x32(a1, bh, acc[1][n]);
      acc[0][n] = mfma16x16x32(a0, bm, acc[0][n]);
      acc[1][n] = mfma16x16x32(a1, bm, acc[1][n]);
      acc[0][n] = mfma16x16x32(a0, bl, acc[0][n]);
      acc[1][n] = mfma16x16x32(a1, bl, acc[1][n]);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): step ks + 1 (B tile and A fragments) landed
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of this step's stage are done
    bar();                                 // so after the barrier the stage may be refilled
    a0 = n0;
    a1 = n1;
  }
  float* out = p.part + (size_t)blockIdx.y * T * EP;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + w * 32 + m * 16 + (lane >> 4) * 4 + r;
      if (t < T) {
#pragma unroll
        for (int n = 0; n < NF; ++n) out[(size_t)t * EP + n * 16 + (lane & 15)] = acc[m][n][r];
      }
    }
}

// router_mfma_kernel with deeper prefetch, for 128 padded experts (every wave
// then issues the same number of weight loads per step, so the waits can be
// counted): the x fragments run DX = 3 steps ahead in a register
// ring, the split weights 2 steps ahead in three LDS stages, and a step waits
// only for its own loads -- not, as router_mfma_kernel does, for everything in
// flight.  Same MFMAs in the same order, so the partials are the same bit for
// bit.
template <int EP>
__global__ __launch_bounds__(512, 1) void router_mfma_pipe_kernel(RouterParams p) {
  constexpr int NF = EP / 16;
  constexpr int ROWS = 3 * EP;          // B rows: split-major (hi, mid, lo)
  constexpr int STAGE = ROWS * 64;      // 32 k (64 bytes) per row
  constexpr int NINS = ROWS / 16;       // 16-row load instructions per stage
  constexpr int NB = NINS / 8;          // of them per wave
  constexpr int NS = 3;                 // weight stages (loads 2 steps ahead)
  constexpr int DX = 3;                 // x fragment ring (loads 3 steps ahead)
  static_assert(NINS % 8 == 0, "every wave issues the same weight loads");
  // loads issued after the later of a step's own (its weights, issued two steps
  // before it, after its x fragments): the next step's x (2), then one step's
  // weights and x (NB + 2)
  constexpr int kWait = 2 + NB + 2;
  static_assert(kWait <= 63, "vmcnt holds at most 63 loads");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = p.T, d = p.d;
  const int t0 = blockIdx.x * 256;
  const int kb = blockIdx.y * p.kslice, ksteps = p.kslice / 32;
  const int kg = lane >> 4;
  const uint16_t* xa0 = p.x + (size_t)min(t0 + w * 32 + (lane & 15), T - 1) * d + kb + kg * 8;
  const uint16_t* xa1 = p.x + (size_t)min(t0 + w * 32 + 16 + (lane & 15), T - 1) * d + kb + kg * 8;
  const int dr = lane >> 2;
  const int dc = (lane & 3) ^ ((dr >> 1) & 3);
  const uint16_t* wsrc = p.wt + (size_t)dr * d + kb + dc * 8;
  const uint32_t bfrag = (uint32_t)((lane & 15) * 64 + ((kg ^ (((lane & 15) >> 1) & 3)) * 16));
  // loads of step ks (clamped to the last step: a refill past the end lands in a
  // stage or ring slot no later step reads)
  auto issue_b = [&](int ks) {
    const int kc = min(ks, ksteps - 1);
    uint8_t* st = smem + (ks % NS) * STAGE;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int q = w + 8 * i;
      __builtin_amdgcn_global_load_lds(MOE_GPTR(wsrc + (size_t)q * 16 * d + kc * 32), MOE_LPTR(st + q * 1024), 16,
                                       0, 0);
    }
  };
  bf16x8_t xr0[DX], xr1[DX];
  auto issue_x = [&](int slot, int ks) {
    const int kc = min(ks, ksteps - 1);
    xr0[slot] = *(const bf16x8_t*)(xa0 + kc * 32);
    xr1[slot] = *(const bf16x8_t*)(xa1 + kc * 32);
  };
  f32x4_t acc[2][NF];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < NF; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // issue order: B(0) x(0) B(1) x(1) x(2), then step j issues B(j + 2) x(j + 3);
  // so after the later of B(j), x(j) come x(j + 1), B(j + 1), x(j + 2) -- kWait loads
  issue_b(0);
  asm volatile("" ::: "memory");
  issue_x(0, 0);
  asm volatile("" ::: "memory");
  issue_b(1);
  asm volatile("" ::: "memory");
  issue_x(1, 1);
  asm volatile("" ::: "memory");
  issue_x(2, 2);
  asm volatile("" ::: "memory");
  auto step = [&](int ks, int slot) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm_r(kWait));  // B(ks) and x(ks) have landed
    __builtin_amdgcn_s_waitcnt(0xC07F);            // this wave's reads of step ks - 1 are done
    bar();                                         // every wave's are: stage (ks + 2) % 3 is free
    __builtin_amdgcn_sched_barrier(0);
    const bf16x8_t a0 = xr0[slot], a1 = xr1[slot];
    issue_b(ks + 2);
    asm volatile("" ::: "memory");
    issue_x(slot, ks + 3);  // the ring slot this step has just taken its fragments from
    asm volatile("" ::: "memory");
    const uint8_t* st = smem + (ks % NS) * STAGE;
#pragma unroll
    for (int n = 0; n < NF; ++n) {
      const bf16x8_t bh = *(const bf16x8_t*)(st + bfrag + (n * 16) * 64);
      const bf16x8_t bm = *(const bf16x8_t*)(st + bfrag + (EP + n * 16) * 64);
      const bf16x8_t bl = *(const bf16x8_t*)(st + bfrag + (2 * EP + n * 16) * 64);
      acc[0][n] = mfma16x16x32(a0, bh, acc[0][n]);
      acc[1][n] = mfma16x16x32(a1, bh, acc[1][n]);
      acc[0][n] = mfma16x16x32(a0, bm, acc[0][n]);
      acc[1][n] = mfma16x16x32(a1, bm, acc[1][n]);
      acc[0][n] = mfma16x16x32(a0, bl, acc[0][n]);
      acc[1][n] = mfma16x16x32(a1, bl, acc[1][n]);
    }
  };
  int ks = 0;
  for (; ks + DX <= ksteps; ks += DX) {
#pragma unroll
    for (int u = 0; u < DX; ++u) step(ks + u, u);
  }
#pragma unroll
  for (int u = 0; u < DX - 1; ++u)
    if (ks + u < ksteps) step(ks + u, u);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm_r(0));  // no load may land in LDS after the block ends
  float* out = p.part + (size_t)blockIdx.y * T * EP;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + w * 32 + m * 16 + (lane >> 4) * 4 + r;
      if (t < T) {
#pragma unroll
        for (int n = 0; n < NF; ++n) out[(size_t)t * EP + n * 16 + (lane & 15)] = acc[m][n][r];
      }
    }
}

// The same partial logits as router_prep_kernel + router_mfma_kernel in one
// launch, block (b, s) taking tokens [256 b, 256 b + 256) over d-slice s.  The block splits its own d-slice of W_r
// (the same exact hi + mid + lo bf16 split, from f32 rows read coalesced along
// the experts) into LDS, laid out as router_mfma_kernel's stages one after the
// other, then runs the same MFMA loop over them in the same order -- so the
// partials are bit-identical to the two-kernel path.
template <int EP>
__global__ __launch_bounds__(512, 1) void router_fused_kernel(const uint16_t* __restrict__ x,
                                                              const float* __restrict__ w, float* __restrict__ part,
                                                              int T, int d, int E, int kslice) {
  constexpr int NF = EP / 16;
  constexpr int ROWS = 3 * EP;          // B rows: split-major (hi, mid, lo)
  constexpr int STAGE = ROWS * 64;      // 32 k (64 bytes) per row
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = blockIdx.y * kslice, ksteps = kslice / 32;
  // ---- split W_r[kb .. kb + kslice)[e] into stage ks = k / 32, row (plane EP + e),
  // 16-byte chunk c = (k % 32) / 8 at slot c ^ ((row >> 1) & 3)
  // (the LDS bound caps kslice * EP at 16384: at most four 8-k chunks per thread,
  // whose 32 loads all go out before any is used)
  // x fragments: rows wv * 32 + lane % 16 (+ 16), k group lane / 16 of each step
  const int kg = lane >> 4;
  const int t0 = blockIdx.x * 256;
  const uint16_t* xa0 = x + (size_t)min(t0 + wv * 32 + (lane & 15), T - 1) * d + kb + kg * 8;
  const uint16_t* xa1 = x + (size_t)min(t0 + wv * 32 + 16 + (lane & 15), T - 1) * d + kb + kg * 8;
  constexpr int kPreSteps = 8;
  bf16x8_t xp0[kPreSteps], xp1[kPreSteps];
  if (ksteps <= kPreSteps) {
#pragma unroll
    for (int ks = 0; ks < kPreSteps; ++ks)
      if (ks < ksteps) {
        xp0[ks] = *(const bf16x8_t*)(xa0 + ks * 32);
        xp1[ks] = *(const bf16x8_t*)(xa1 + ks * 32);
      }
  }
  const int nchunks = kslice / 8;
  float wv8[4][8];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int it = tid + u * 512;
    const int e = it % EP, kc = it / EP;  // experts fastest: the f32 reads coalesce
#pragma unroll
    for (int q = 0; q < 8; ++q)
      wv8[u][q] = (it < nchunks * EP && e < E) ? w[(size_t)(kb + kc * 8 + q) * E + e] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int it = tid + u * 512;
    if (it >= nchunks * EP) break;
    const int e = it % EP, kc = it / EP;
    uint32_t hi[4], mid[4], lo[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t h2 = 0, m2 = 0, l2 = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float v = wv8[u][q * 2 + h];
        const uint16_t bh = f32_to_bf16_rne(v);
        const float r1 = v - bf16_bits_to_f32(bh);
        const uint16_t bm = f32_to_bf16_rne(r1);
        const float r2 = r1 - bf16_bits_to_f32(bm);
        const uint16_t bl = f32_to_bf16_rne(r2);
        h2 |= (uint32_t)bh << (16 * h);
        m2 |= (uint32_t)bm << (16 * h);
        l2 |= (uint32_t)bl << (16 * h);
      }
      hi[q] = h2; mid[q] = m2; lo[q] = l2;
    }
    const int ks = kc / 4, c = kc % 4;
    uint8_t* st = smem + (size_t)ks * STAGE;
#pragma unroll
    for (int pl = 0; pl < 3; ++pl) {
      const int row = pl * EP + e;
      const uint4 v = pl == 0 ? make_uint4(hi[0], hi[1], hi[2], hi[3])
                    : pl == 1 ? make_uint4(mid[0], mid[1], mid[2], mid[3])
                              : make_uint4(lo[0], lo[1], lo[2], lo[3]);
      *(uint4*)(st + row * 64 + ((c ^ ((row >> 1) & 3)) * 16)) = v;
    }
  }
  // ---- the MFMA loop of router_mfma_kernel over the resident stages
  const uint32_t bfrag = (uint32_t)((lane & 15) * 64 + ((kg ^ (((lane & 15) >> 1) & 3)) * 16));
  f32x4_t acc[2][NF];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < NF; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto step = [&](int ks, const bf16x8_t& a0, const bf16x8_t& a1) {
    const uint8_t* st = smem + (size_t)ks * STAGE;
#pragma unroll
    for (int n = 0; n < NF; ++n) {
      const bf16x8_t bh = *(const bf16x8_t*)(st + bfrag + (n * 16) * 64);
      const bf16x8_t bm = *(const bf16x8_t*)(st + bfrag + (EP + n * 16) * 64);
      const bf16x8_t bl = *(const bf16x8_t*)(st + bfrag + (2 * EP + n * 16) * 64);
      acc[0][n] = mfma16x16x32(a0, bh, acc[0][n]);
      acc[1][n] = mfma16x16x32(a1, bh, acc[1][n]);
      acc[0][n] = mfma16x16x32(a0, bm, acc[0][n]);
      acc[1][n] = mfma16x16x32(a1, bm, acc[1][n]);
      acc[0][n] = mfma16x16x32(a0, bl, acc[0][n]);
      acc[1][n] = mfma16x16x32(a1, bl, acc[1][n]);
    }
  };
  if (ksteps <= kPreSteps) {
    // the slice's x fragments were all requested before the split (above): the
    // loop waits for memory once, not once per step
    __syncthreads();  // the split slice is in LDS
#pragma unroll
    for (int ks = 0; ks < kPreSteps; ++ks)
      if (ks < ksteps) step(ks, xp0[ks], xp1[ks]);
  } else {
    bf16x8_t a0 = *(const bf16x8_t*)xa0, a1 = *(const bf16x8_t*)xa1;
    __syncthreads();  // the split slice is in LDS
    for (int ks = 0; ks < ksteps; ++ks) {
      bf16x8_t n0 = a0, n1 = a1;
      if (ks + 1 < ksteps) {
        n0 = *(const bf16x8_t*)(xa0 + (ks + 1) * 32);
        n1 = *(const bf16x8_t*)(xa1 + (ks + 1) * 32);
      }
      step(ks, a0, a1);
      a0 = n0;
      a1 = n1;
    }
  }
  float* out = part + (size_t)blockIdx.y * T * EP;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + wv * 32 + m * 16 + (lane >> 4) * 4 + r;
      if (t < T) {
#pragma unroll
        for (int n = 0; n < NF; ++n) out[(size_t)t * EP + n * 16 + (lane & 15)] = acc[m][n][r];
      }
    }
}

// one wave per token: z = sum of the d-slice partials in order, then route_token.
// The partials of the lane's experts are requested PB slices at a time and
// then added in slice order: PB = 32 for small batches (one memory round trip
// for a decode batch), 8 otherwise (fewer registers, more waves per SIMD).
template <int EPL, int PB>
__global__ __launch_bounds__(256) void topk_kernel(RouteLaunch a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int S = a.split, EP = a.ep, T = a.T, E = a.E;
  const size_t st = (size_t)T * EP;
  float zv[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) zv[i] = 0.f;
  for (int s0 = 0; s0 < S; s0 += PB) {
    float v[EPL][PB];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      const float* pe = a.part + (size_t)t * EP + e;
#pragma unroll
      for (int q = 0; q < PB; ++q) v[i][q] = (s0 + q < S && e < E) ? pe[(size_t)(s0 + q) * st] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i)
#pragma unroll
      for (int q = 0; q < PB; ++q)
        if (s0 + q < S) zv[i] += v[i][q];
  }
  route_token<EPL>(a, t, lane, [&](int e) { return zv[(e - lane) >> 6]; });
}

// Small batches (at most 256 tokens): one block of four waves per token.  Wave
// v adds the slices [S v / 4, S (v + 1) / 4) of its lanes' experts -- all of
// them requested at once, one memory round trip -- and the four sums meet in
// LDS, added in wave order; wave 0 then runs route_token.  (With one wave per
// token a 64-slice decode batch makes two round trips: 128 loads per lane are
// more than the 63 the load counter holds.)
template <int EPL>
__global__ __launch_bounds__(256) void topk_quarters_kernel(RouteLaunch a) {
  constexpr int PQ = 16;  // slices per wave requested together (S <= 64 takes one round)
  __shared__ float zq[4][EPL][64];
  const int lane = threadIdx.x & 63;
  const int v = threadIdx.x >> 6;
  const int t = blockIdx.x;
  const int S = a.split, EP = a.ep, T = a.T, E = a.E;
  const size_t st = (size_t)T * EP;
  const int s_lo = S * v / 4, s_hi = S * (v + 1) / 4;
  float zv[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) zv[i] = 0.f;
  for (int s0 = s_lo; s0 < s_hi; s0 += PQ) {
    float x[EPL][PQ];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      const float* pe = a.part + (size_t)t * EP + e;
#pragma unroll
      for (int q = 0; q < PQ; ++q) x[i][q] = (s0 + q < s_hi && e < E) ? pe[(size_t)(s0 + q) * st] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i)
#pragma unroll
      for (int q = 0; q < PQ; ++q)
        if (s0 + q < s_hi) zv[i] += x[i][q];
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) zq[v][i][lane] = zv[i];
  __syncthreads();
  if (v != 0) return;
  float z[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) z[i] = ((zq[0][i][lane] + zq[1][i][lane]) + zq[2][i][lane]) + zq[3][i][lane];
  route_token<EPL>(a, t, lane, [&](int e) { return z[(e - lane) >> 6]; });
}

// the top-k pass over the router's partials: four waves per token for small
// batches, one otherwise
template <int EP>
moe_status launch_topk(const RouteLaunch& a, hipStream_t s) {
  int tok = begin_launch("route_topk", s);
  if (a.T <= 256)
    hipLaunchKernelGGL((topk_quarters_kernel<(EP + 63) / 64>), dim3((unsigned)a.T), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((topk_kernel<(EP + 63) / 64, 8>), dim3((unsigned)ceil_div(a.T, 4)), dim3(256), 0, s, a);
  return end_launch(tok, s);
}

template <int EP>
moe_status launch_mfma_route(const RouteLaunch& a, hipStream_t s) {
  const int kslice = a.d / a.split;
  const size_t fused_lds = (size_t)(kslice / 32) * 3 * EP * 64;
  if (fused_lds <= kFusedRouterLds && (size_t)kslice * EP <= 16384) {
    // more than 64 KB of dynamic LDS needs the attribute, set once per device
    // (a repeat after a race between threads is harmless)
    static std::atomic<bool> lds_set[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
      return fail(MOE_ERR_HIP, "hipGetDevice failed or device id out of range");
    if (!lds_set[dev].load(std::memory_order_acquire)) {
      if (hipFuncSetAttribute((const void*)router_fused_kernel<EP>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kFusedRouterLds) != hipSuccess)
        return fail(MOE_ERR_HIP, "hipFuncSetAttribute(router_fused_kernel) failed");
      lds_set[dev].store(true, std::memory_order_release);
    }
    int tok = begin_launch("router_mfma", s);
    hipLaunchKernelGGL(router_fused_kernel<EP>, dim3((unsigned)ceil_div(a.T, 256), a.split), dim3(512), fused_lds, s,
                       (const uint16_t*)a.x, a.w_router, a.part, a.T, a.d, a.E, kslice);
    moe_status st = end_launch(tok, s);
    if (st != MOE_OK) return st;
    return launch_topk<EP>(a, s);
  }
  int tok = begin_launch("router_prep", s);
  hipLaunchKernelGGL(router_prep_kernel, dim3(a.d / 32, (unsigned)ceil_div(EP, 64)), dim3(256), 0, s,
                     a.w_router, a.wt, a.d, a.E, EP);
  moe_status st = end_launch(tok, s);
  if (st != MOE_OK) return st;
  RouterParams rp{(const uint16_t*)a.x, a.wt, a.part, a.T, a.d, a.d / a.split};
  tok = begin_launch("router_mfma", s);
  // 128 padded experts: the pipelined loop (skewed fp8 layer 57.1 -> 52.4 us); at
  // 256 its 256 VGPRs spill and it ran slower (89 -> 105 us), so that width keeps
  // the plain loop
  if constexpr (EP == 128)
    hipLaunchKernelGGL(router_mfma_pipe_kernel<EP>, dim3((unsigned)ceil_div(a.T, 256), a.split), dim3(512), 0, s, rp);
  else
    hipLaunchKernelGGL(router_mfma_kernel<EP>, dim3((unsigned)ceil_div(a.T, 256), a.split), dim3(512), 0, s, rp);
  st = end_launch(tok, s);
  if (st != MOE_OK) return st;
  return launch_topk<EP>(a, s);
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
  if (a.act_dtype != MOE_BF16) return dispatch<false>(a, s);
  switch (a.ep) {
    case 16: return launch_mfma_route<16>(a, s);
    case 32: return launch_mfma_route<32>(a, s);
    case 64: return launch_mfma_route<64>(a, s);
    case 128: return launch_mfma_route<128>(a, s);
    default: return launch_mfma_route<256>(a, s);
  }
}

void route_plan(int T, int d, int E, int act_dtype, int* ep, int* split) {
  if (act_dtype != MOE_BF16) { *ep = 0; *split = 0; return; }
  int p = 16;
  while (p < E) p *= 2;
  *ep = p;
  // about one block per CU: token blocks x d-slices, the slice a multiple of 32
  const int tblocks = (int)ceil_div(std::max(T, 1), 256);
  const int target = std::max(1, device_cu_count() / tblocks);
  const int steps = d / 32;
  // at least four 32-wide steps per slice (two for at most 256 tokens): the
  // top-k pass then has few partials to add; for a decode batch two steps per
  // slice (64 slices at d = 4096) made the router 10.4 -> 6.7 us and the top-k
  // 7.5 -> 9.0 us (kernel trace), against four
  int sp = std::min(target, std::max(1, T <= 256 ? steps / 2 : steps / 4));
  while (steps % sp) --sp;
  *split = sp;
}

}  // namespace moe
