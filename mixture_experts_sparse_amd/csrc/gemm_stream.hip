// Grouped expert GEMM for expert groups of few rows: streams the weights.
//
// Same computation and tile walk as gemm.hip (page "MoE sparse activation:
// principles and engineering practice" (kapook.pages.dev), s4.2 expert fusion
// and s4.2 quantisation; page "GPT-4 has 1.8T parameters but uses 2% per token"
// (mlqm.cn), s3.3 SwiGLU).  When an expert holds tens of rows (capacity-limited
// or decode batches) the pass is bound by reading the weights, so the kernel is
// built around streaming them once at full bandwidth:
//
//  * block = 4 waves x 64 weight rows (256 per block), tile = BM = 16 MF rows
//    of the expert (MF = 2 or 4), of which only the live 16-row groups (those
//    holding rows of the expert) are loaded and multiplied;
//  * each wave loads its own weight rows straight into registers, 128 k per
//    step (one 128-byte line per fp8 row, two per bf16 row, half a line per
//    INT4 row), into a ring of register sets PD steps ahead;
//  * the BM activation rows of a step are shared through LDS, filled by direct
//    global -> LDS loads DA >= PD steps ahead into DA + 1 stages, 16-byte chunk
//    c of row r at slot c ^ (r & 15) so the fragment reads are conflict-free.
//    The load counter retires loads in issue order, so a step waiting for its
//    activations also waits for every weight load issued before them: the
//    weights are only as far ahead in flight as the activations are;
//  * a weight row's bytes of a step are read in 64-byte parts, lane group g
//    (lane / 16) taking bytes 16 g .. 16 g + 15 of each, so every load
//    instruction covers whole half lines; the k values that gives each lane
//    group in each sub-step (kchunk) are read from the activations too, so
//    every MFMA pairs equal k;
//  * fp8 (OCP e4m3fn) codes become bf16 in registers
//    (v_cvt_scalef32_pk_bf16_fp8, exact) and row scales multiply the f32
//    accumulators in the epilogue;
//  * group-wise INT4 (128 weights per group, each with its own scale and zero
//    point; w = scale * (q - zero)): one K step is exactly one group, so a
//    lane's 32 codes of a step are one 16-byte load and every weight row adds
//    one 32-bit group word (fp16 scale | zero << 16) per step.  A code q becomes
//    the bf16 number 128 + q by byte permutes alone (0x4300 | q: exponent 2^7,
//    q in the mantissa -- exact), the step's products are summed on the MFMA
//    into a per-step accumulator t, one more MFMA against a fragment of ones
//    gives the row sums of the activations, and
//        acc += scale * (t - (128 + zero) * rowsum)
//    applies the group's parameters once per step and output element.
#include <algorithm>
#include <type_traits>

#include "grouped.h"

namespace moe {
namespace {

#define MOE_GPTR(p) ((const __attribute__((address_space(1))) void*)(p))
#define MOE_LPTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kKS = 128;   // k per step

constexpr unsigned vmcnt_imm(int n) { return 0x0F70u | (unsigned)(n & 15) | ((unsigned)(n >> 4) << 14); }
constexpr unsigned kLgkm0 = 0xC07Fu;  // lgkmcnt(0) alone

__device__ __forceinline__ void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Keeps the compiler from reordering memory operations across this point: the
// waits count loads in flight newest first, so load groups must issue in the
// order written.
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

enum { WT_BF16 = 0, WT_FP8 = 1, WT_INT4 = 2 };

template <int WT, int MF>
struct Plan {
  static constexpr int RAW = WT == WT_BF16 ? 4 : WT == WT_FP8 ? 2 : 1;  // 16-byte loads per fragment per step
  static constexpr int NQ = WT == WT_INT4 ? 1 : 0;                       // group words per fragment per step
  static constexpr int STEP_BYTES = WT == WT_BF16 ? 256 : WT == WT_FP8 ? 128 : 64;  // per weight row
  // weight prefetch distance (registers allowing) and activation distance
  static constexpr int PD = WT == WT_BF16 ? 1 : (MF >= 4 ? 2 : 3);
  static constexpr int DA = PD < 2 ? 2 : PD;
};

struct StreamParams {
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

template <int WT, int NF>
struct WSet {
  uint4 w[NF][Plan<WT, 2>::RAW];
  uint32_t q[NF][1];  // INT4 group words (unused otherwise)
};

// 8 bf16 of sub-step s from a lane's raw weight registers of one fragment
template <int WT>
__device__ __forceinline__ bf16x8_t b_frag(const uint4 (&raw)[Plan<WT, 2>::RAW], int s) {
  if constexpr (WT == WT_BF16) {
    return __builtin_bit_cast(bf16x8_t, raw[s]);  // load s: 8 bf16
  } else if constexpr (WT == WT_FP8) {
    const uint4 q = raw[s >> 1];  // 16 codes; sub-step s uses half s & 1
    const uint32_t lo = (s & 1) ? q.z : q.x, hi = (s & 1) ? q.w : q.y;
    uint4 o;
    o.x = fp8x2_to_bf16x2<false>(lo);
    o.y = fp8x2_to_bf16x2<true>(lo);
    o.z = fp8x2_to_bf16x2<false>(hi);
    o.w = fp8x2_to_bf16x2<true>(hi);
    return __builtin_bit_cast(bf16x8_t, o);
  } else {
    const uint4 c = raw[0];  // 32 codes; sub-step s uses word s
    return int4_frag(s == 0 ? c.x : s == 1 ? c.y : s == 2 ? c.z : c.w);
  }
}

// The k chunk (8 values: 16 bytes of a bf16 activation row) that lane group
// g4 holds in sub-step s.  A lane's weight bytes of a step are its 16-byte
// loads u at byte 64 u + 16 g4 of the row's step, so each load instruction
// covers 64 contiguous bytes of its 16 rows (one half line each, every byte
// used by that one instruction); sub-step s takes bf16: load s; fp8: half
// s & 1 of load s >> 1; INT4: word s of the one load.  The activation
// fragments are read at the same k, so each MFMA still pairs equal k.
template <int WT>
__device__ __forceinline__ int kchunk(int g4, int s) {
  if constexpr (WT == WT_BF16) return 4 * s + g4;
  else if constexpr (WT == WT_FP8) return 8 * (s >> 1) + 2 * g4 + (s & 1);
  else return 4 * g4 + s;
}

template <bool GATED, int WT, int MF>
__global__ __launch_bounds__(256, 2) void gemm_stream_kernel(StreamParams p) {
  using PL = Plan<WT, MF>;
  constexpr int BM = 16 * MF;
  constexpr int NF = 4;                    // n-fragments (16 weight rows) per wave
  constexpr int AROW = kKS * 2;            // 256 bytes per activation row
  constexpr int ASTAGE = BM * AROW;
  constexpr int PD = PL::PD, DA = PL::DA, R = PD + 1, NST = DA + 1;
  constexpr int NB = NF * (PL::RAW + PL::NQ);  // weight loads per wave per step
  __shared__ __attribute__((aligned(1024))) uint8_t As[NST * ASTAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = p.K, N = p.N, ksteps = K / kKS;
  const int total = p.n_tiles * p.tp[p.groups];
  const int G8 = gridDim.x >> 3, xcd = blockIdx.x & 7, jb = blockIdx.x >> 3;
  const int chunk = (total + 7) >> 3;
  const int lend = min(total, (xcd + 1) * chunk);
  const int g4 = lane >> 4, r16 = lane & 15;
  const size_t RB = (size_t)K * PL::STEP_BYTES / kKS;  // bytes per weight row
  const size_t KG = (size_t)K / kKS;                    // group words per weight row
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));

  // activation DMA: instruction i of wave w covers rows 16 i + 4 w .. + 3 (so the
  // first i instructions of every wave fill the first i 16-row groups); lane: row
  // (lane >> 4), slot (lane & 15) <- chunk slot ^ (row & 15)
  const int dma_r = lane >> 4;
  // fragment read for sub-step s, m-fragment i: row 16 i + r16, chunk kchunk(g4, s)
  const uint32_t afrag = (uint32_t)(r16 * AROW);

  for (int L = xcd * chunk + jb; L < lend; L += G8) {
    const TileRef tr = map_tile(L, p.n_tiles, p.groups, BM, p.tp, p.goff);
    const int g = tr.g;
    // rows past the group's end repeat its last row; with a gather map the rows
    // come straight from the token matrix (offsets checked to fit 32 bits)
    const uint8_t* a_base = (const uint8_t*)p.A + (p.gather ? 0 : (size_t)tr.row0 * K * 2);
    uint32_t a_off[MF];
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      const int r = 16 * i + 4 * w + dma_r;
      const int c = (lane & 15) ^ (r & 15);
      const int rr = min(r, tr.rows - 1);
      const uint32_t src = p.gather ? (uint32_t)p.gather[tr.row0 + rr] : (uint32_t)rr;
      a_off[i] = src * (uint32_t)K * 2u + (uint32_t)(c * 16);
    }
    // this lane's weight rows (one per n-fragment), at byte 16 g4 of each 64-byte part
    const uint8_t* b_row[NF];
    const uint32_t* q_row[NF];
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      int wrow;
      const void* base;
      const void* qbase;
      if (GATED) {  // fragments 0,1: gate rows; 2,3: the matching up rows
        wrow = tr.nt * 128 + w * 32 + (j & 1) * 16 + r16;
        base = (j < 2) ? p.B0 : p.B1;
        qbase = (j < 2) ? p.S0 : p.S1;
      } else {
        wrow = tr.nt * 256 + w * 64 + j * 16 + r16;
        base = p.B0;
        qbase = p.S0;
      }
      const size_t row = (size_t)g * N + wrow;
      b_row[j] = (const uint8_t*)base + row * RB + (size_t)g4 * 16;
      q_row[j] = (const uint32_t*)qbase + row * KG;
    }
    // the activation loads of step ks: the NL live 16-row groups only
    auto issue_a = [&](int ks, auto nl) {
      constexpr int NL = decltype(nl)::value;
      uint8_t* st = As + (ks % NST) * ASTAGE;
      const uint32_t kb = (uint32_t)min(ks, ksteps - 1) * AROW;
#pragma unroll
      for (int i = 0; i < NL; ++i)
        __builtin_amdgcn_global_load_lds(MOE_GPTR(a_base + a_off[i] + kb), MOE_LPTR(st + (4 * i + w) * 1024),
                                         16, 0, 0);
    };
    auto load_w = [&](WSet<WT, NF>& d, int ks) {
      const int kc = min(ks, ksteps - 1);
#pragma unroll
      for (int j = 0; j < NF; ++j)
#pragma unroll
        for (int u = 0; u < PL::RAW; ++u)
          d.w[j][u] = *(const uint4*)(b_row[j] + (size_t)kc * PL::STEP_BYTES + u * 64);
      if constexpr (PL::NQ > 0) {
#pragma unroll
        for (int j = 0; j < NF; ++j) d.q[j][0] = q_row[j][kc];
      }
    };

    // the tile, for NL live 16-row groups (rows past the group's end fill the last
    // group; whole groups past it are neither loaded nor multiplied)
    auto run_tile = [&](auto nl) {
      constexpr int NL = decltype(nl)::value;
      // loads issued after the last one step k needs (weights of k from step k - PD,
      // activations of k from step k - DA, each step issuing weights then activations)
      constexpr int kWaitBody = (DA > PD ? NL : 0) + (PD - 1) * (NL + NB);
      // past the main loop the weight prefetches feed no step, the compiler drops
      // them, and only the activation loads remain behind
      constexpr int kWaitTail = (DA > PD ? NL : 0) + (PD - 1) * NL;
      static_assert(kWaitBody <= 63, "vmcnt holds at most 63 loads");
      f32x4_t acc[NL][NF];
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j) acc[i][j] = zero4;
      WSet<WT, NF> ring[R];

      // one K step: weights of `ks` in cur; weights of ks + PD requested into nxt
      auto step = [&](int ks, const WSet<WT, NF>& cur, WSet<WT, NF>& nxt, auto tail) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(decltype(tail)::value ? kWaitTail : kWaitBody));
        // this wave's LDS reads of step ks - 1 are complete before the barrier:
        // after it, another wave may refill that stage
        __builtin_amdgcn_s_waitcnt(kLgkm0);
        block_sync();
        __builtin_amdgcn_sched_barrier(0);  // nothing of this step moves above the waits
        load_w(nxt, ks + PD);
        issue_fence();
        issue_a(ks + DA, nl);
        issue_fence();
        const uint8_t* st = As + (ks % NST) * ASTAGE;
        f32x4_t t[NL][NF], rs[NL];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t slot = (uint32_t)((kchunk<WT>(g4, s) ^ r16) * 16);
          bf16x8_t af[NL], bf[NF];
#pragma unroll
          for (int i = 0; i < NL; ++i) af[i] = *(const bf16x8_t*)(st + afrag + i * 16 * AROW + slot);
#pragma unroll
          for (int j = 0; j < NF; ++j) bf[j] = b_frag<WT>(cur.w[j], s);
#pragma unroll
          for (int i = 0; i < NL; ++i) {
            if constexpr (WT == WT_INT4) {
              rs[i] = mfma16x16x32(af[i], ones, s == 0 ? zero4 : rs[i]);
#pragma unroll
              for (int j = 0; j < NF; ++j) t[i][j] = mfma16x16x32(af[i], bf[j], s == 0 ? zero4 : t[i][j]);
            } else {
#pragma unroll
              for (int j = 0; j < NF; ++j) acc[i][j] = mfma16x16x32(af[i], bf[j], acc[i][j]);
            }
          }
        }
        if constexpr (WT == WT_INT4) {
#pragma unroll
          for (int j = 0; j < NF; ++j) {
            const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)(cur.q[j][0] & 0xFFFFu));
            const float c = (float)(128u + ((cur.q[j][0] >> 16) & 15u));
#pragma unroll
            for (int i = 0; i < NL; ++i)
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(sc, fmaf(-c, rs[i][r], t[i][j][r]), acc[i][j][r]);
          }
        }
      };

      block_sync();  // the previous tile's stages are free
      // issue order: step j (j = -DA .. -1 here, then 0, 1, ...) issues the weights
      // of j + PD and then the activations of j + DA
#pragma unroll
      for (int j = -DA; j < 0; ++j) {
        if (j + PD >= 0) load_w(ring[j + PD], j + PD);
        issue_fence();
        issue_a(j + DA, nl);
        issue_fence();
      }
      // step k computes from set k % R and refills set (k + PD) % R, the one step
      // k - 1 used; whole rounds of R steps, then the remaining steps
      int ks = 0;
      for (; ks + R <= ksteps; ks += R) {
#pragma unroll
        for (int u = 0; u < R; ++u) step(ks + u, ring[u], ring[(u + PD) % R], std::false_type{});
      }
#pragma unroll
      for (int u = 0; u < R - 1; ++u)
        if (ks + u < ksteps) step(ks + u, ring[u], ring[(u + PD) % R], std::true_type{});
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load may land in a stage after this tile

      // ---- epilogue (rows past the group's end are not stored)
      const int rq = g4 * 4;
      if (GATED) {
        uint16_t* h = (uint16_t*)p.out;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int f = tr.nt * 128 + w * 32 + j * 16 + r16;
          float sg = 1.f, su = 1.f;
          if constexpr (WT == WT_FP8) {
            sg = ((const float*)p.S0)[(size_t)g * N + f];
            su = ((const float*)p.S1)[(size_t)g * N + f];
          }
#pragma unroll
          for (int i = 0; i < NL; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int m = i * 16 + rq + r;
              if (m < tr.rows)
                h[(size_t)(tr.row0 + m) * N + f] = f32_to_bf16_rne(silu_f32(acc[i][j][r] * sg) * (acc[i][j + 2][r] * su));
            }
        }
      } else {
        float* y = (float*)p.out;
#pragma unroll
        for (int j = 0; j < NF; ++j) {
          const int n = tr.nt * 256 + w * 64 + j * 16 + r16;
          float sd = 1.f;
          if constexpr (WT == WT_FP8) sd = ((const float*)p.S0)[(size_t)g * N + n];
#pragma unroll
          for (int i = 0; i < NL; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int m = i * 16 + rq + r;
              if (m < tr.rows) y[(size_t)(tr.row0 + m) * N + n] = acc[i][j][r] * sd;
            }
        }
      }
    };
    const int nl = min(MF, (tr.rows + 15) >> 4);
    if (nl >= MF) run_tile(std::integral_constant<int, MF>{});
    else if (MF == 4 && nl == 3) run_tile(std::integral_constant<int, (MF > 3 ? 3 : 1)>{});
    else if (nl == 2) run_tile(std::integral_constant<int, (MF > 2 ? 2 : 1)>{});
    else run_tile(std::integral_constant<int, 1>{});
  }
}

template <bool GATED, int WT>
void launch_t(const StreamParams& p, int mf, int64_t grid, hipStream_t s) {
  if (mf == 2) hipLaunchKernelGGL((gemm_stream_kernel<GATED, WT, 2>), dim3(grid), dim3(256), 0, s, p);
  else hipLaunchKernelGGL((gemm_stream_kernel<GATED, WT, 4>), dim3(grid), dim3(256), 0, s, p);
}

}  // namespace

moe_status launch_gemm_stream(const GemmLaunch& a, const int32_t* goff, const int32_t* tp, int bm, hipStream_t s) {
  StreamParams p{a.A, a.B0, a.B1, a.S0, a.S1, a.out, goff, tp, a.groups, a.K, a.N, 0, a.gather};
  p.n_tiles = a.gated ? a.N / 128 : a.N / 256;
  const int64_t upper = (ceil_div(a.max_rows, bm) + a.groups) * p.n_tiles;
  int64_t grid = std::min<int64_t>(upper, (int64_t)device_cu_count() * 2);
  grid = ceil_div(grid, 8) * 8;
  if (grid <= 0) return MOE_OK;
  const int wt = a.w_dtype == MOE_FP8_E4M3FN ? WT_FP8 : a.w_dtype == MOE_INT4 ? WT_INT4 : WT_BF16;
  const int mf = bm / 16;
  if (wt == WT_INT4 && mf != 2) return fail(MOE_ERR_UNSUPPORTED, "INT4 weights take 32-row tiles");
  static const char* const kNames[2][2][3] = {
      {{"gemm_down_bf16", "gemm_down_fp8", "gemm_down_int4"},
       {"gemm_gate_up_bf16", "gemm_gate_up_fp8", "gemm_gate_up_int4"}},
      {{"shared_down_bf16", "shared_down_fp8", "shared_down_int4"},
       {"shared_gate_up_bf16", "shared_gate_up_fp8", "shared_gate_up_int4"}}};
  int tok = begin_launch(kNames[a.shared][a.gated][wt], s);
  if (a.gated) {
    if (wt == WT_BF16) launch_t<true, WT_BF16>(p, mf, grid, s);
    else if (wt == WT_FP8) launch_t<true, WT_FP8>(p, mf, grid, s);
    else hipLaunchKernelGGL((gemm_stream_kernel<true, WT_INT4, 2>), dim3(grid), dim3(256), 0, s, p);
  } else {
    if (wt == WT_BF16) launch_t<false, WT_BF16>(p, mf, grid, s);
    else if (wt == WT_FP8) launch_t<false, WT_FP8>(p, mf, grid, s);
    else hipLaunchKernelGGL((gemm_stream_kernel<false, WT_INT4, 2>), dim3(grid), dim3(256), 0, s, p);
  }
  return end_launch(tok, s);
}

}  // namespace moe
