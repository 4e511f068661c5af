// Grouped expert GEMM for expert groups of at most 16 rows (decode batches):
// the four waves of a block split K.
//
// Same computation as gemm.hip (page "MoE sparse activation: principles and
// engineering practice" (kapook.pages.dev), s4.2 expert fusion and s4.2
// quantisation; page "GPT-4 has 1.8T parameters but uses 2% per token"
// (mlqm.cn), s3.3 SwiGLU).  When every expert holds a handful of rows the pass
// is one read of the touched experts' weights, and what limits it is how many
// weight bytes the chip keeps in flight.  With 256 weight rows per block and
// all of K in one wave chain (gemm_stream.hip), a decode batch that touches
// 15 experts makes 180 gate/up tiles -- fewer blocks than CUs, one wave per
// SIMD, a 32-step chain of dependent loads per wave.  Here:
//
//  * tile = 16 rows x 64 weight rows (gate/up: 32 gate + the 32 matching up
//    rows; down: 64 output columns), one MFMA fragment of rows, four 16-row
//    weight fragments: four times the blocks of the streaming kernel;
//  * the block's four waves take consecutive quarters of K and run without a
//    block barrier: each wave streams its quarter of the 64 weight rows into
//    registers and its quarter of the 16 activation rows into an LDS ring of
//    its own by direct global -> LDS loads, both PD steps ahead, so it only ever
//    waits for its own loads;
//  * at the end the four partial accumulators meet in LDS (fixed order: wave
//    0 + 1 + 2 + 3) and the epilogue writes h (gate/up: silu(gate) * up, bf16)
//    or y (f32);
//  * weights bf16, fp8 e4m3fn (exact conversion to bf16, row scale in the
//    epilogue) or group-wise INT4 (one 128-weight group per step: codes as bf16
//    128 + q, the step's products and an MFMA row sum against ones, then
//    acc += scale * (t - (128 + zero) * rowsum)).
#include <algorithm>
#include <type_traits>

#include "grouped.h"

namespace moe {
namespace {

#define MOE_GPTR(p) ((const __attribute__((address_space(1))) void*)(p))
#define MOE_LPTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kKS = 128;                // k per step
constexpr int kBM = 16;                 // rows per tile
constexpr int kNF = 4;                  // 16-row weight fragments per tile
constexpr int kAROW = kKS * 2;          // bytes of one activation row per step

constexpr unsigned vmcnt_imm(int n) { return 0x0F70u | (unsigned)(n & 15) | ((unsigned)(n >> 4) << 14); }
constexpr unsigned kLgkm0 = 0xC07Fu;  // lgkmcnt(0) alone

// keeps load groups in the order written (the waits count loads newest first)
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

// blocks per CU the registers and LDS are sized for, and the prefetch distances
#ifndef KS_OCC
#define KS_OCC 2
#endif
#ifndef KS_PD_BF16
#define KS_PD_BF16 2
#endif
#ifndef KS_PD_FP8
#define KS_PD_FP8 3
#endif
#ifndef KS_PD_INT4
#define KS_PD_INT4 4
#endif
// with at most 4 rows per expert (capacity 1-4: decode) only those rows are staged
#ifndef KS_PD4_FP8
#define KS_PD4_FP8 3
#endif
#ifndef KS_PD4_INT4
#define KS_PD4_INT4 4
#endif

enum { WT_BF16 = 0, WT_FP8 = 1, WT_INT4 = 2 };

template <int WT, int AR>
struct Codec {
  static constexpr int RAW = WT == WT_BF16 ? 4 : WT == WT_FP8 ? 2 : 1;  // 16-byte loads per fragment per step
  static constexpr int NQ = WT == WT_INT4 ? 1 : 0;                       // group words per fragment per step
  static constexpr int STEP_BYTES = WT == WT_BF16 ? 256 : WT == WT_FP8 ? 128 : 64;  // per weight row
  // prefetch distance D in steps, for the weights (registers) and the activations
  // (D + 1 LDS stages per wave) alike: the waits count loads in issue order, so
  // the weights are only ever as far ahead as the activations issued beside them
  static constexpr int PD = WT == WT_BF16 ? KS_PD_BF16
                            : WT == WT_FP8  ? (AR == 4 ? KS_PD4_FP8 : KS_PD_FP8)
                                            : (AR == 4 ? KS_PD4_INT4 : KS_PD_INT4);
  static constexpr int NB = kNF * (RAW + NQ);                            // weight loads per wave per step
};

struct KsplitParams {
  const void* A;
  const void* B0;
  const void* B1;
  const void* S0;  // fp8: f32 row scales [groups][N]; INT4: uint32 group words [groups][N][K/128]
  const void* S1;
  void* out;
  const int32_t* goff;
  const int32_t* tp;
  int groups, K, N, n_tiles;
  const int32_t* gather;  // A row r is A[gather[r]], or null
};

template <int WT>
struct WSet {
  uint4 w[kNF][Codec<WT, 16>::RAW];
  uint32_t q[kNF][Codec<WT, 16>::NQ > 0 ? Codec<WT, 16>::NQ : 1];
};

// 8 bf16 of sub-step s from a lane's raw weight registers of one fragment
template <int WT>
__device__ __forceinline__ bf16x8_t b_frag(const uint4 (&raw)[Codec<WT, 16>::RAW], int s) {
  if constexpr (WT == WT_BF16) {
    return __builtin_bit_cast(bf16x8_t, raw[s]);
  } else if constexpr (WT == WT_FP8) {
    const uint4 q = raw[s >> 1];
    const uint32_t lo = (s & 1) ? q.z : q.x, hi = (s & 1) ? q.w : q.y;
    uint4 o;
    o.x = fp8x2_to_bf16x2<false>(lo);
    o.y = fp8x2_to_bf16x2<true>(lo);
    o.z = fp8x2_to_bf16x2<false>(hi);
    o.w = fp8x2_to_bf16x2<true>(hi);
    return __builtin_bit_cast(bf16x8_t, o);
  } else {
    const uint4 c = raw[0];
    return int4_frag(s == 0 ? c.x : s == 1 ? c.y : s == 2 ? c.z : c.w);
  }
}

// AR: activation rows staged per tile, 16 (every tile) or 4 (tiles of at most 4
// rows: fragment row r reads staged row r & 3, so rows 4-15 of the MFMA repeat
// rows 0-3 and are never stored)
template <bool GATED, int WT, int AR>
__global__ __launch_bounds__(256, KS_OCC) void gemm_ksplit_kernel(KsplitParams p) {
  using CD = Codec<WT, AR>;
  constexpr int PD = CD::PD, R = PD + 1, NB = CD::NB;
  constexpr int NST = PD + 1;  // activation stages per wave
  constexpr int kASTAGE = AR * kAROW;   // bytes per stage
  constexpr int kAINS = kASTAGE / 1024; // 1 KB direct-to-LDS loads per wave per step
  static_assert(PD >= 2 && (PD - 1) * (NB + kAINS) <= 63, "vmcnt holds at most 63 loads");
  static_assert(4 * NST * kASTAGE * KS_OCC <= 160 * 1024, "LDS of the resident blocks");
  static_assert(4 * NST * kASTAGE >= 4 * kNF * 4 * 64 * 4, "the partial sums meet in the stage memory");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * NST * kASTAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = p.K, N = p.N, ksteps = K / kKS;
  // this wave's steps [k0, k0 + nk)
  const int q4 = (ksteps + 3) >> 2;
  const int k0 = min(ksteps, w * q4);
  const int nk = min(ksteps, k0 + q4) - k0;
  const int total = p.n_tiles * p.tp[p.groups];
  const int G8 = gridDim.x >> 3, xcd = blockIdx.x & 7, jb = blockIdx.x >> 3;
  const int chunk = (total + 7) >> 3;
  const int lend = min(total, (xcd + 1) * chunk);
  const int g4 = lane >> 4, r16 = lane & 15;
  const size_t RB = (size_t)K * CD::STEP_BYTES / kKS;  // bytes per weight row
  const size_t KG = (size_t)K / kKS;                    // group words per weight row
  uint8_t* As = smem + w * (NST * kASTAGE);
  const uint32_t afrag = (uint32_t)((r16 % AR) * kAROW);
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));

  for (int L = xcd * chunk + jb; L < lend; L += G8) {
    const TileRef tr = map_tile(L, p.n_tiles, p.groups, kBM, p.tp, p.goff);
    const int g = tr.g;
    f32x4_t acc[kNF];
#pragma unroll
    for (int j = 0; j < kNF; ++j) acc[j] = zero4;

    if (nk > 0) {
      // activations: load i covers rows 4 i .. 4 i + 3; lane: row 4 i + lane / 16,
      // 16-byte chunk slot (lane & 15) <- chunk slot ^ (row & 15); rows past the
      // group's end repeat its last row
      const uint8_t* a_base = (const uint8_t*)p.A + (p.gather ? 0 : (size_t)tr.row0 * K * 2);
      uint32_t a_off[kAINS];
#pragma unroll
      for (int i = 0; i < kAINS; ++i) {
        const int r = i * 4 + (lane >> 4);
        const int c = (lane & 15) ^ (r & 15);
        const int rr = min(r, tr.rows - 1);
        const uint32_t src = p.gather ? (uint32_t)p.gather[tr.row0 + rr] : (uint32_t)rr;
        a_off[i] = src * (uint32_t)K * 2u + (uint32_t)(c * 16);
      }
      // weights: fragment j's row for this lane; lane group g4 holds k = 32 g4 .. + 31 of a step
      const uint8_t* b_row[kNF];
      const uint32_t* q_row[kNF];
#pragma unroll
      for (int j = 0; j < kNF; ++j) {
        int wrow;
        const void* base;
        const void* qbase;
        if (GATED) {  // fragments 0,1: gate rows; 2,3: the matching up rows
          wrow = tr.nt * 32 + (j & 1) * 16 + r16;
          base = (j < 2) ? p.B0 : p.B1;
          qbase = (j < 2) ? p.S0 : p.S1;
        } else {
          wrow = tr.nt * 64 + j * 16 + r16;
          base = p.B0;
          qbase = p.S0;
        }
        const size_t row = (size_t)g * N + wrow;
        b_row[j] = (const uint8_t*)base + row * RB + (size_t)g4 * (CD::STEP_BYTES / 4);
        q_row[j] = (const uint32_t*)qbase + row * KG;
      }
      // Steps past this wave's last (prefetches near the end) still issue their
      // loads -- the waits count them -- but every lane reads one common address,
      // so each such instruction costs one request and no bandwidth.
      auto issue_a = [&](int k) {  // k: local step
        uint8_t* st = As + (k % NST) * kASTAGE;
        const bool live = k < nk;
        const uint32_t kb = (uint32_t)(k0 + min(k, nk - 1)) * kAROW;
#pragma unroll
        for (int i = 0; i < kAINS; ++i)
          __builtin_amdgcn_global_load_lds(MOE_GPTR(live ? a_base + a_off[i] + kb : (const uint8_t*)p.A),
                                           MOE_LPTR(st + i * 1024), 16, 0, 0);
      };
      auto load_w = [&](WSet<WT>& d, int k) {
        const bool live = k < nk;
        const int kc = k0 + min(k, nk - 1);
#pragma unroll
        for (int j = 0; j < kNF; ++j)
#pragma unroll
          for (int u = 0; u < CD::RAW; ++u)
            d.w[j][u] = *(const uint4*)(live ? b_row[j] + (size_t)kc * CD::STEP_BYTES + u * 16 : (const uint8_t*)p.B0);
        if constexpr (CD::NQ > 0) {
#pragma unroll
          for (int j = 0; j < kNF; ++j) d.q[j][0] = live ? q_row[j][kc] : *(const uint32_t*)p.S0;
        }
      };

      WSet<WT> ring[R];
      // one step: weights of local step k in cur, those of k + PD requested into nxt
      auto step = [&](int k, const WSet<WT>& cur, WSet<WT>& nxt, auto tail) {
        constexpr bool kTail = decltype(tail)::value;
        // landed: all but the newest loads -- the PD - 1 steps issued since this
        // step's (weights then activations, each).  Past the main loop the weight
        // prefetches feed no step and the compiler removes them, so there only
        // the activations of those steps are counted.
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((PD - 1) * (kAINS + (kTail ? 0 : NB))));
        // this wave's reads of step k - 1 are done before step k + PD refills that stage
        __builtin_amdgcn_s_waitcnt(kLgkm0);
        __builtin_amdgcn_sched_barrier(0);  // nothing of this step moves above the waits
        load_w(nxt, k + PD);
        issue_fence();
        issue_a(k + PD);
        issue_fence();
        const uint8_t* st = As + (k % NST) * kASTAGE;
        f32x4_t t[kNF], rs = zero4;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t slot = (uint32_t)(((4 * g4 + s) ^ (r16 % AR)) * 16);
          const bf16x8_t af = *(const bf16x8_t*)(st + afrag + slot);
          bf16x8_t bf[kNF];
#pragma unroll
          for (int j = 0; j < kNF; ++j) bf[j] = b_frag<WT>(cur.w[j], s);
          if constexpr (WT == WT_INT4) {
            rs = mfma16x16x32(af, ones, s == 0 ? zero4 : rs);
#pragma unroll
            for (int j = 0; j < kNF; ++j) t[j] = mfma16x16x32(af, bf[j], s == 0 ? zero4 : t[j]);
          } else {
#pragma unroll
            for (int j = 0; j < kNF; ++j) acc[j] = mfma16x16x32(af, bf[j], acc[j]);
          }
        }
        if constexpr (WT == WT_INT4) {
#pragma unroll
          for (int j = 0; j < kNF; ++j) {
            const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)(cur.q[j][0] & 0xFFFFu));
            const float c = (float)(128u + ((cur.q[j][0] >> 16) & 15u));
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[j][r] = fmaf(sc, fmaf(-c, rs[r], t[j][r]), acc[j][r]);
          }
        }
      };

      // issue order: weights then activations of steps 0 .. PD-1; then step k
      // issues those of step k + PD
#pragma unroll
      for (int u = 0; u < PD; ++u) {
        load_w(ring[u], u);
        issue_fence();
        issue_a(u);
        issue_fence();
      }
      // step k computes from set k % R and refills set (k + PD) % R = (k - 1) % R
      int k = 0;
      for (; k + R <= nk; k += R) {
#pragma unroll
        for (int u = 0; u < R; ++u) step(k + u, ring[u], ring[(u + PD) % R], std::false_type{});
      }
#pragma unroll
      for (int u = 0; u < R - 1; ++u)
        if (k + u < nk) step(k + u, ring[u], ring[(u + PD) % R], std::true_type{});
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load may land in LDS after this point
      __builtin_amdgcn_s_waitcnt(kLgkm0);
    }

    // ---- the four partial sums meet in LDS (the stages are free once every wave is
    // here).  __syncthreads: LDS writes complete before the barrier, unlike a bare s_barrier
    __syncthreads();
    float* red = (float*)smem;  // [wave][fragment][r][lane]
#pragma unroll
    for (int j = 0; j < kNF; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[((w * kNF + j) * 4 + r) * 64 + lane] = acc[j][r];
    __syncthreads();
    auto total_of = [&](int j, int r) {
      float v = red[((0 * kNF + j) * 4 + r) * 64 + lane];
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) v += red[((ww * kNF + j) * 4 + r) * 64 + lane];
      return v;
    };
    const int rq = g4 * 4;  // lane holds rows rq .. rq + 3 of the tile, column r16 of each fragment
    if (GATED) {
      if (w < 2) {  // wave j: gate fragment j and up fragment j + 2
        const int j = w;
        const int f = tr.nt * 32 + j * 16 + r16;
        float sg = 1.f, su = 1.f;
        if constexpr (WT == WT_FP8) {
          sg = ((const float*)p.S0)[(size_t)g * N + f];
          su = ((const float*)p.S1)[(size_t)g * N + f];
        }
        uint16_t* h = (uint16_t*)p.out;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = rq + r;
          if (m < tr.rows)
            h[(size_t)(tr.row0 + m) * N + f] = f32_to_bf16_rne(silu_f32(total_of(j, r) * sg) * (total_of(j + 2, r) * su));
        }
      }
    } else {  // wave j: fragment j
      const int j = w;
      const int n = tr.nt * 64 + j * 16 + r16;
      float sd = 1.f;
      if constexpr (WT == WT_FP8) sd = ((const float*)p.S0)[(size_t)g * N + n];
      float* y = (float*)p.out;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = rq + r;
        if (m < tr.rows) y[(size_t)(tr.row0 + m) * N + n] = total_of(j, r) * sd;
      }
    }
    __syncthreads();  // the reduction area is read before the next tile's loads refill it
  }
}

}  // namespace

moe_status launch_gemm_ksplit(const GemmLaunch& a, const int32_t* goff, const int32_t* tp, hipStream_t s) {
  KsplitParams p{a.A, a.B0, a.B1, a.S0, a.S1, a.out, goff, tp, a.groups, a.K, a.N, 0, a.gather};
  p.n_tiles = a.gated ? a.N / 32 : a.N / 64;
  const int64_t upper = (ceil_div(a.max_rows, kBM) + a.groups) * p.n_tiles;
  int64_t grid = std::min<int64_t>(upper, (int64_t)device_cu_count() * KS_OCC);
  grid = ceil_div(grid, 8) * 8;  // the XCD mapping wants a multiple of 8
  if (grid <= 0) return MOE_OK;
  const int wt = a.w_dtype == MOE_FP8_E4M3FN ? WT_FP8 : a.w_dtype == MOE_INT4 ? WT_INT4 : WT_BF16;
  // every group has at most 4 rows (capacity 1-4): stage only those
  const bool few = a.group_rows_max >= 0 && a.group_rows_max <= 4 && wt != WT_BF16;
  static const char* const kNames[2][2][3] = {
      {{"gemm_down_bf16", "gemm_down_fp8", "gemm_down_int4"},
       {"gemm_gate_up_bf16", "gemm_gate_up_fp8", "gemm_gate_up_int4"}},
      {{"shared_down_bf16", "shared_down_fp8", "shared_down_int4"},
       {"shared_gate_up_bf16", "shared_gate_up_fp8", "shared_gate_up_int4"}}};
  int tok = begin_launch(kNames[a.shared][a.gated][wt], s);
  const dim3 gd((unsigned)grid), bd(256);
  auto go = [&](auto gated, auto wtag, auto ar) {
    hipLaunchKernelGGL((gemm_ksplit_kernel<decltype(gated)::value, decltype(wtag)::value, decltype(ar)::value>), gd,
                       bd, 0, s, p);
  };
  using T1 = std::true_type;
  using F1 = std::false_type;
  using B = std::integral_constant<int, WT_BF16>;
  using F8 = std::integral_constant<int, WT_FP8>;
  using I4 = std::integral_constant<int, WT_INT4>;
  using A16 = std::integral_constant<int, 16>;
  using A4 = std::integral_constant<int, 4>;
  if (a.gated) {
    if (wt == WT_BF16) go(T1{}, B{}, A16{});
    else if (wt == WT_FP8) { if (few) go(T1{}, F8{}, A4{}); else go(T1{}, F8{}, A16{}); }
    else { if (few) go(T1{}, I4{}, A4{}); else go(T1{}, I4{}, A16{}); }
  } else {
    if (wt == WT_BF16) go(F1{}, B{}, A16{});
    else if (wt == WT_FP8) { if (few) go(F1{}, F8{}, A4{}); else go(F1{}, F8{}, A16{}); }
    else { if (few) go(F1{}, I4{}, A4{}); else go(F1{}, I4{}, A16{}); }
  }
  return end_launch(tok, s);
}

}  // namespace moe
