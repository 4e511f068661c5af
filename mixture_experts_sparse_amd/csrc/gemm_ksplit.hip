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
// in K steps per weight type
constexpr int kOcc = 2;
constexpr int kPdBf16 = 2;
constexpr int kPdFp8 = 3;
constexpr int kPdInt4 = 4;
// with at most 4 rows per expert (capacity 1-4: decode) only those rows are staged
constexpr int kPd4Fp8 = 3;
constexpr int kPd4Int4 = 4;

enum { WT_BF16 = 0, WT_FP8 = 1, WT_INT4 = 2 };

template <int WT, int AR>
struct Codec {
  static constexpr int RAW = WT == WT_BF16 ? 4 : WT == WT_FP8 ? 2 : 1;  // 16-byte loads per fragment per step
  static constexpr int NQ = WT == WT_INT4 ? 1 : 0;                       // group words per fragment per step
  static constexpr int STEP_BYTES = WT == WT_BF16 ? 256 : WT == WT_FP8 ? 128 : 64;  // per weight row
  // prefetch distance D in steps, for the weights (registers) and the activations
  // (D + 1 LDS stages per wave) alike: the waits count loads in issue order, so
  // the weights are only ever as far ahead as the activations issued beside them
  static constexpr int PD = WT == WT_BF16 ? kPdBf16
                            : WT == WT_FP8  ? (AR == 4 ? kPd4Fp8 : kPdFp8)
                                            : (AR == 4 ? kPd4Int4 : kPdInt4);
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

// The k chunk (8 values: 16 bytes of a bf16 activation row) that lane group
// g4 holds in sub-step s.  A lane's weight bytes of a step are its 16-byte
// loads u at byte 64 u + 16 g4 of the row's step, so each load instruction
// covers 64 contiguous bytes of its 16 rows; sub-step s takes bf16: load s;
// fp8: half s & 1 of load s >> 1; INT4: word s of the one load.  The
// activation fragments are read at the same k, so each MFMA pairs equal k.
template <int WT>
__device__ __forceinline__ int kchunk(int g4, int s) {
  if constexpr (WT == WT_BF16) return 4 * s + g4;
  else if constexpr (WT == WT_FP8) return 8 * (s >> 1) + 2 * g4 + (s & 1);
  else return 4 * g4 + s;
}

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

// Fragment j's weight row for this lane -- gate/up: fragments 0,1 gate rows,
// 2,3 the matching up rows; down: four consecutive 16-row fragments -- at byte
// 16 g4 of each 64-byte part of a step, and that row's INT4 group words.
template <bool GATED>
__device__ __forceinline__ void tile_weight_rows(const KsplitParams& p, const TileRef& tr, int r16, int g4,
                                                 size_t RB, size_t KG, const uint8_t* (&b_row)[kNF],
                                                 const uint32_t* (&q_row)[kNF]) {
#pragma unroll
  for (int j = 0; j < kNF; ++j) {
    int wrow;
    const void* base;
    const void* qbase;
    if (GATED) {
      wrow = tr.nt * 32 + (j & 1) * 16 + r16;
      base = (j < 2) ? p.B0 : p.B1;
      qbase = (j < 2) ? p.S0 : p.S1;
    } else {
      wrow = tr.nt * 64 + j * 16 + r16;
      base = p.B0;
      qbase = p.S0;
    }
    const size_t row = (size_t)tr.g * p.N + wrow;
    b_row[j] = (const uint8_t*)base + row * RB + (size_t)g4 * 16;
    q_row[j] = (const uint32_t*)qbase + row * KG;
  }
}

// The output column of this lane's epilogue rows (gate/up: h column, written by
// waves 0 and 1; down: y column of fragment w), whose fp8 row scales apply.
template <bool GATED>
__device__ __forceinline__ int tile_out_col(const TileRef& tr, int w, int r16) {
  return GATED ? tr.nt * 32 + (w & 1) * 16 + r16 : tr.nt * 64 + w * 16 + r16;
}

// A tile's four partial sums meet in `red` ([wave][fragment][r][lane]; fixed
// order wave 0 + 1 + 2 + 3) and the tile's outputs are written: gate/up, waves
// 0 and 1 write h = silu(gate sc0) * (up sc1) for fragment pair (w, w + 2);
// down, wave w writes y = fragment w times sc0.  sync(): a block barrier after
// this wave's LDS operations, taken after the sums are written and after they
// are read.
template <bool GATED, typename Sync>
__device__ __forceinline__ void tile_epilogue(const KsplitParams& p, const TileRef& tr, const f32x4_t (&acc)[kNF],
                                              float* red, int w, int lane, float sc0, float sc1, Sync sync) {
#pragma unroll
  for (int j = 0; j < kNF; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[((w * kNF + j) * 4 + r) * 64 + lane] = acc[j][r];
  sync();
  auto total_of = [&](int j, int r) {
    float v = red[((0 * kNF + j) * 4 + r) * 64 + lane];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) v += red[((ww * kNF + j) * 4 + r) * 64 + lane];
    return v;
  };
  const int rq = (lane >> 4) * 4;  // lane holds rows rq .. rq + 3 of the tile
  const int col = tile_out_col<GATED>(tr, w, lane & 15);
  if (GATED) {
    if (w < 2) {
      uint16_t* h = (uint16_t*)p.out;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = rq + r;
        if (m < tr.rows)
          h[(size_t)(tr.row0 + m) * p.N + col] = f32_to_bf16_rne(silu_f32(total_of(w, r) * sc0) * (total_of(w + 2, r) * sc1));
      }
    }
  } else {
    float* y = (float*)p.out;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = rq + r;
      if (m < tr.rows) y[(size_t)(tr.row0 + m) * p.N + col] = total_of(w, r) * sc0;
    }
  }
  sync();
}

// AR: activation rows staged per tile, 16 (every tile) or 4 (tiles of at most 4
// rows: fragment row r reads staged row r & 3, so rows 4-15 of the MFMA repeat
// rows 0-3 and are never stored)
template <bool GATED, int WT, int AR>
__global__ __launch_bounds__(256, kOcc) void gemm_ksplit_kernel(KsplitParams p) {
  using CD = Codec<WT, AR>;
  constexpr int PD = CD::PD, R = PD + 1, NB = CD::NB;
  constexpr int NST = PD + 1;  // activation stages per wave
  constexpr int kASTAGE = AR * kAROW;   // bytes per stage
  constexpr int kAINS = kASTAGE / 1024; // 1 KB direct-to-LDS loads per wave per step
  static_assert(PD >= 2 && (PD - 1) * (NB + kAINS) <= 63, "vmcnt holds at most 63 loads");
  static_assert(4 * NST * kASTAGE * kOcc <= 160 * 1024, "LDS of the resident blocks");
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
      const uint8_t* b_row[kNF];
      const uint32_t* q_row[kNF];
      tile_weight_rows<GATED>(p, tr, r16, g4, RB, KG, b_row, q_row);
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
            d.w[j][u] = *(const uint4*)(live ? b_row[j] + (size_t)kc * CD::STEP_BYTES + u * 64 : (const uint8_t*)p.B0);
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
          const uint32_t slot = (uint32_t)((kchunk<WT>(g4, s) ^ (r16 % AR)) * 16);
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

    // ---- the four partial sums meet in LDS, in the stage memory: free once every
    // wave is here.  __syncthreads: LDS writes complete before the barrier,
    // unlike a bare s_barrier
    __syncthreads();
    float sc0 = 1.f, sc1 = 1.f;
    if constexpr (WT == WT_FP8) {
      const size_t at = (size_t)g * N + tile_out_col<GATED>(tr, w, r16);
      sc0 = ((const float*)p.S0)[at];
      sc1 = GATED ? ((const float*)p.S1)[at] : sc0;
    }
    // the second barrier: the reduction area is read before the next tile's loads refill it
    tile_epilogue<GATED>(p, tr, acc, (float*)smem, w, lane, sc0, sc1, [] { __syncthreads(); });
  }
}

// Tiles of at most 4 rows with K split evenly, INT4 weights (decode): the
// tile work of gemm_ksplit_kernel<GATED, WT_INT4, 4>, but each wave's load
// stream runs on across the block's tiles.  A wave's steps over its tiles form
// one sequence, and PD steps ahead of the step it computes it requests the
// weights and activations of the step PD later -- in the next tile once this
// one has no more -- so the prefetch never drains at a tile boundary; the
// partial sums meet in an LDS area of their own while the next tile's loads
// are in flight.  Needs K / 128 = 4 nk steps with nk a multiple of PD + 1 (a
// step's ring slot and LDS stage are then the same in every tile).  Every
// vector load of the stream is one the waits count: the tile table and the
// gathered token indices come through scalar loads.
typedef const __attribute__((address_space(4))) int32_t* cint_ptr;

// A block barrier after this wave's LDS operations have completed -- and
// nothing else: __syncthreads would also wait for every load in flight, which
// here are the next tile's prefetches.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kLgkm0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ TileRef map_tile_scalar(int L, int n_tiles, int groups, int bm, cint_ptr tp,
                                                   cint_ptr goff) {
  L = __builtin_amdgcn_readfirstlane(L);
  const int g = tp[groups + 1 + L / n_tiles];
  const int mt = tp[g + 1] - tp[g];
  const int local = L - tp[g] * n_tiles;
  TileRef r;
  r.g = g;
  r.nt = local / mt;
  r.row0 = goff[g] + (local % mt) * bm;
  r.rows = min(bm, goff[g + 1] - r.row0);
  return r;
}

template <bool GATED, int WT, int PD>
__global__ __launch_bounds__(256, kOcc) void gemm_ksplit_pipe_kernel(KsplitParams p) {
  static_assert(WT == WT_INT4 || WT == WT_FP8, "INT4 or fp8 weights");
  constexpr int AR = 4;
  using CD = Codec<WT, AR>;
  constexpr int R = PD + 1;
  constexpr int NS = kNF * CD::RAW + 1;            // loads of a step: 16-byte weight loads + the activations
  // + at a chunk's first step: INT4, one group-word load per fragment; fp8, the
  // row scales of the tile (read for real only when the chunk starts a tile)
  constexpr int NQ = WT == WT_INT4 ? kNF : (GATED ? 2 : 1);
  constexpr int kASTAGE = AR * kAROW;              // 1 KB: one direct-to-LDS load per step
  constexpr int kRED = 4 * kNF * 4 * 64 * 4;       // the four waves' partial sums
  static_assert(kASTAGE == 1024, "one activation load per step");
  static_assert(R <= 4, "a chunk's group words: one per lane group");
  static_assert(PD >= 2 && (PD - 1) * NS + NQ <= 63, "vmcnt holds at most 63 loads");
  static_assert(kOcc * (4 * R * kASTAGE + kRED) <= 160 * 1024, "LDS of the resident blocks");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * R * kASTAGE + kRED];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = p.K, N = p.N;
  const int nk = K / kKS / 4;  // steps per wave per tile (the host checks 4 nk = K / 128, nk % R == 0)
  const int k0 = w * nk;
  cint_ptr tp = (cint_ptr)p.tp;
  cint_ptr goff = (cint_ptr)p.goff;
  cint_ptr gat = (cint_ptr)p.gather;
  const int total = p.n_tiles * tp[p.groups];
  const int G8 = gridDim.x >> 3, xcd = blockIdx.x & 7, jb = blockIdx.x >> 3;
  const int chunk = (total + 7) >> 3;
  const int lend = min(total, (xcd + 1) * chunk);
  const int L0 = xcd * chunk + jb;
  if (L0 >= lend) return;  // the whole block: no tile
  const int n_units = (lend - L0 + G8 - 1) / G8;
  const int g4 = lane >> 4, r16 = lane & 15;
  const size_t RB = (size_t)K * CD::STEP_BYTES / kKS;
  const size_t KG = (size_t)K / kKS;
  uint8_t* As = smem + w * (R * kASTAGE);
  float* red = (float*)(smem + 4 * R * kASTAGE);  // [wave][fragment][r][lane]
  const uint32_t afrag = (uint32_t)((r16 & 3) * kAROW);
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));

  // ---- the issue side: the tile whose steps are being requested (past the
  // block's last tile every lane reads one common address: one request each)
  const uint8_t* a_src;
  const uint8_t* b_row[kNF];
  const uint32_t* q_row[kNF];
  const float* sc_at[2];  // fp8: where this lane's output-row scales of the tile are
  bool ilive;
  auto set_issue = [&](int iu) {
    ilive = iu < n_units;
    const TileRef tr = map_tile_scalar(L0 + min(iu, n_units - 1) * G8, p.n_tiles, p.groups, kBM, tp, goff);
    // activations: lane -> row lane / 16 (rows past the group's end repeat its
    // last row), 16-byte chunk slot lane % 16 <- chunk slot ^ row
    const int r = lane >> 4;
    const int c = (lane & 15) ^ r;
    uint32_t src;
    if (p.gather) {
      const int s0 = gat[tr.row0];
      const int s1 = gat[tr.row0 + min(1, tr.rows - 1)];
      const int s2 = gat[tr.row0 + min(2, tr.rows - 1)];
      const int s3 = gat[tr.row0 + min(3, tr.rows - 1)];
      src = (uint32_t)(r == 0 ? s0 : r == 1 ? s1 : r == 2 ? s2 : s3);
    } else {
      src = (uint32_t)(tr.row0 + min(r, tr.rows - 1));
    }
    a_src = (const uint8_t*)p.A + (size_t)src * K * 2 + c * 16;
    tile_weight_rows<GATED>(p, tr, r16, g4, RB, KG, b_row, q_row);
    if constexpr (WT == WT_FP8) {  // the row scales of this lane's epilogue column
      const size_t at = (size_t)tr.g * N + tile_out_col<GATED>(tr, w, r16);
      sc_at[0] = (const float*)p.S0 + at;
      sc_at[1] = GATED ? (const float*)p.S1 + at : sc_at[0];
    }
  };
  // one step's loads, into ring slot / LDS stage `slot`: the weights of local
  // step k of the issue tile; at a chunk's first step, INT4: the chunk's group
  // words spread over the lanes (lane group g4 < R: the word of step k + g4 of
  // its fragment row) -- one load per fragment per chunk instead of one per
  // step; fp8: the tile's row scales when the chunk starts the tile, else a
  // load of the common address (no branch: the waits stay exact); then the
  // activations
  uint4 wr[R][kNF][CD::RAW];
  uint32_t qd[kNF];
  float sl[2];
  auto issue = [&](int slot, int k, auto chunk_start) {
    const int kc = k0 + k;
#pragma unroll
    for (int j = 0; j < kNF; ++j)
#pragma unroll
      for (int u = 0; u < CD::RAW; ++u)
        wr[slot][j][u] =
            *(const uint4*)(ilive ? b_row[j] + (size_t)kc * CD::STEP_BYTES + u * 64 : (const uint8_t*)p.B0);
    if constexpr (decltype(chunk_start)::value) {
      if constexpr (WT == WT_INT4) {
#pragma unroll
        for (int j = 0; j < kNF; ++j) qd[j] = ilive ? q_row[j][kc + min(g4, R - 1)] : *(const uint32_t*)p.S0;
      } else {
#pragma unroll
        for (int i = 0; i < NQ; ++i) sl[i] = *(ilive && k == 0 ? sc_at[i] : (const float*)p.S0);
      }
    }
    issue_fence();
    __builtin_amdgcn_global_load_lds(MOE_GPTR(ilive ? a_src + (size_t)kc * kAROW : (const uint8_t*)p.A),
                                     MOE_LPTR(As + slot * kASTAGE), 16, 0, 0);
    issue_fence();
  };

  set_issue(0);
  issue(0, 0, std::true_type{});
#pragma unroll
  for (int u = 1; u < PD; ++u) issue(u, u, std::false_type{});

  float st_sc[2] = {1.f, 1.f};  // fp8: the current tile's row scales
  for (int cu = 0; cu < n_units; ++cu) {
    const TileRef tr = map_tile_scalar(L0 + cu * G8, p.n_tiles, p.groups, kBM, tp, goff);
    f32x4_t acc[kNF];
#pragma unroll
    for (int j = 0; j < kNF; ++j) acc[j] = zero4;
    for (int kb = 0; kb < nk; kb += R) {
      uint32_t qw[R][kNF];  // INT4: this chunk's group word of each step and fragment
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int k = kb + u;
        // landed: all but the loads of the PD - 1 steps requested after this one
        // (one of them a chunk's first step, with its extra loads, unless this
        // step or the one before starts a chunk); epilogue stores between them
        // only make the wait stricter
        if (u >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm((PD - 1) * NS + NQ));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm((PD - 1) * NS));
        // this wave's reads of the previous step are done before its stage is refilled
        __builtin_amdgcn_s_waitcnt(kLgkm0);
        __builtin_amdgcn_sched_barrier(0);
        if (u == 0) {
          // what landed with the chunk's first step: INT4, the chunk's words to every
          // lane of a row (qd is then free for the next chunk's, requested at u == 1);
          // fp8, in the tile's first chunk, the tile's scales (likewise)
          if constexpr (WT == WT_INT4) {
#pragma unroll
            for (int v = 0; v < R; ++v)
#pragma unroll
              for (int j = 0; j < kNF; ++j) qw[v][j] = (uint32_t)__shfl((int)qd[j], v * 16 + r16);
          } else {
#pragma unroll
            for (int i = 0; i < NQ; ++i) st_sc[i] = kb == 0 ? sl[i] : st_sc[i];
          }
        }
        if (u == 1 && kb + R == nk) set_issue(cu + 1);  // k + PD == nk: the next tile's steps from here
        const int kn = k + PD < nk ? k + PD : k + PD - nk;
        // (u + PD) % R == 0 exactly when u == 1: the requested step starts a chunk
        if (u == 1) issue((u + PD) % R, kn, std::true_type{});
        else issue((u + PD) % R, kn, std::false_type{});
        const uint8_t* st = As + u * kASTAGE;
        f32x4_t t[kNF], rs = zero4;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t slot = (uint32_t)((kchunk<WT>(g4, s) ^ (r16 & 3)) * 16);
          const bf16x8_t af = *(const bf16x8_t*)(st + afrag + slot);
          if constexpr (WT == WT_INT4) {
            rs = mfma16x16x32(af, ones, s == 0 ? zero4 : rs);
#pragma unroll
            for (int j = 0; j < kNF; ++j) t[j] = mfma16x16x32(af, b_frag<WT>(wr[u][j], s), s == 0 ? zero4 : t[j]);
          } else {
#pragma unroll
            for (int j = 0; j < kNF; ++j) acc[j] = mfma16x16x32(af, b_frag<WT>(wr[u][j], s), acc[j]);
          }
        }
        if constexpr (WT == WT_INT4) {
#pragma unroll
          for (int j = 0; j < kNF; ++j) {
            const uint32_t q = qw[u][j];
            const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)(q & 0xFFFFu));
            const float c = (float)(128u + ((q >> 16) & 15u));
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[j][r] = fmaf(sc, fmaf(-c, rs[r], t[j][r]), acc[j][r]);
          }
        }
      }
    }

    // ---- the four partial sums meet in their own LDS area (the stages hold the
    // next tile's loads in flight)
    tile_epilogue<GATED>(p, tr, acc, red, w, lane, st_sc[0], st_sc[1], [] { lds_barrier(); });
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load may land in LDS after the block ends
}

}  // namespace

moe_status launch_gemm_ksplit(const GemmLaunch& a, const int32_t* goff, const int32_t* tp, hipStream_t s) {
  KsplitParams p{a.A, a.B0, a.B1, a.S0, a.S1, a.out, goff, tp, a.groups, a.K, a.N, 0, a.gather};
  p.n_tiles = a.gated ? a.N / 32 : a.N / 64;
  const int64_t upper = (ceil_div(a.max_rows, kBM) + a.groups) * p.n_tiles;
  int64_t grid = std::min<int64_t>(upper, (int64_t)device_cu_count() * kOcc);
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
  // INT4 or fp8 tiles of at most 4 rows, K split evenly: the load stream runs across tiles
  const int ksteps = a.K / kKS;
  const int nk = ksteps / 4;
  if (few && ksteps % 4 == 0 && nk > 0 && (nk % 4 == 0 || nk % 3 == 0)) {
    auto pipe = [&](auto gated, auto wtag) {
      constexpr bool G = decltype(gated)::value;
      constexpr int WTv = decltype(wtag)::value;
      if (nk % 4 == 0) hipLaunchKernelGGL((gemm_ksplit_pipe_kernel<G, WTv, 3>), gd, bd, 0, s, p);
      else hipLaunchKernelGGL((gemm_ksplit_pipe_kernel<G, WTv, 2>), gd, bd, 0, s, p);
    };
    using I4p = std::integral_constant<int, WT_INT4>;
    using F8p = std::integral_constant<int, WT_FP8>;
    if (a.gated) { if (wt == WT_INT4) pipe(std::true_type{}, I4p{}); else pipe(std::true_type{}, F8p{}); }
    else { if (wt == WT_INT4) pipe(std::false_type{}, I4p{}); else pipe(std::false_type{}, F8p{}); }
    return end_launch(tok, s);
  }
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
