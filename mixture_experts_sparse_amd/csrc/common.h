// Internal helpers shared by the HIP kernels of the MoE layer (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---------------------------------------------------------------- vectors
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

constexpr int kWave = 64;

// bf16 <-> f32 (bit-level; bf16 is the top half of an f32)
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}
__host__ __device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// MFMA 16x16x32 bf16 -> f32.  Lane l supplies A[m = l%16][8 k-values of group l/16]
// and B[the same 8 k-values][n = l%16]; it receives D[m = 4*(l/16) + r][n = l%16]
// in element r.  A and B use one k-mapping, so the sum over k is exact whatever
// order the hardware assigns within a group.
__device__ __forceinline__ f32x4_t mfma16x16x32(const bf16x8_t& a, const bf16x8_t& b,
                                                const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Two OCP e4m3fn codes (bytes 0,1 of `packed`, or bytes 2,3 when HIGH) -> two bf16;
// exact (fp8 values are a subset of bf16), hardware conversion with unit scale.
template <bool HIGH>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t packed) {
  bf16x2_t v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(packed, 1.0f, HIGH);
  return __builtin_bit_cast(uint32_t, v);
}

// 16 e4m3fn codes (one uint4) -> 16 bf16 (two uint4), element order preserved.
__device__ __forceinline__ void fp8x16_to_bf16x16(const uint4& q, uint4& lo, uint4& hi) {
  lo.x = fp8x2_to_bf16x2<false>(q.x);
  lo.y = fp8x2_to_bf16x2<true>(q.x);
  lo.z = fp8x2_to_bf16x2<false>(q.y);
  lo.w = fp8x2_to_bf16x2<true>(q.y);
  hi.x = fp8x2_to_bf16x2<false>(q.z);
  hi.y = fp8x2_to_bf16x2<true>(q.z);
  hi.z = fp8x2_to_bf16x2<false>(q.w);
  hi.w = fp8x2_to_bf16x2<true>(q.w);
}

// 8 INT4 codes (one 32-bit word: even k in the low nibble of each byte) as the
// bf16 values 128 + q, in k order.  v_perm_b32 picks bytes of {S0, S1} (S1 =
// bytes 0-3, S0 = bytes 4-7) by selector.
__device__ __forceinline__ bf16x8_t int4_frag(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu;                   // q0 q2 q4 q6 (bytes)
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;            // q1 q3 q5 q7
  const uint32_t x = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // q0 q1 q2 q3
  const uint32_t y = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // q4 q5 q6 q7
  constexpr uint32_t C = 0x43434343u;                    // bf16 128 = 0x4300
  uint4 o;
  o.x = __builtin_amdgcn_perm(C, x, 0x04010400u);        // [q0, 43, q1, 43]
  o.y = __builtin_amdgcn_perm(C, x, 0x04030402u);        // [q2, 43, q3, 43]
  o.z = __builtin_amdgcn_perm(C, y, 0x04010400u);
  o.w = __builtin_amdgcn_perm(C, y, 0x04030402u);
  return __builtin_bit_cast(bf16x8_t, o);
}

// silu(g) = g / (1 + e^-g), with the hardware reciprocal (1 ulp): its result is
// rounded to bf16 (or compared at 1e-4 in fp32) right after, and the correctly
// rounded division costs about ten instructions per element in the epilogues
__device__ __forceinline__ float silu_f32(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// ---------------------------------------------------------------- host side
// Record a launch for the profiling hook; returns an index for end_launch().
int begin_launch(const char* name, hipStream_t s);
// Checks hipGetLastError() after a launch; closes the profiling bracket.
moe_status end_launch(int token, hipStream_t s);
// Thread-local error message setter.
moe_status fail(moe_status st, const char* fmt, ...);
// Number of compute units on the current device (cached per device).
int device_cu_count();

// Integer helpers
__host__ __device__ constexpr inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ constexpr inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------- kernel launchers
// Implemented in the .hip files; every launcher returns MOE_OK or MOE_ERR_HIP.
struct RouteLaunch {
  const void* x; const float* w_router; const float* bias; const float* gumbel_u;
  float* logits; int32_t* topk_idx; float* topk_w;
  int T, d, E, k, score, renormalize, bias_mode, act_dtype;
  float tau;
  // bf16 path: padded expert count, d-split, and workspace buffers
  int fb = 0;               // fallback experts written after the top-k (topk_idx has k + fb columns)
  int n_groups = 0, topk_groups = 0;  // group-limited routing (0 = off)
  int ep = 0, split = 0;
  uint16_t* wt = nullptr;   // [3][ep][d] split router weights
  float* part = nullptr;    // [split][T][ep] logit partials
};
moe_status launch_route(const RouteLaunch& a, hipStream_t s);
// Router geometry for bf16 activations (ep = 0 for the fp32 path): padded expert
// count (16 .. 256) and the number of d-slices.  Depends on the device's CU count.
void route_plan(int T, int d, int E, int act_dtype, int* ep, int* split);

// Permutation geometry: pairs are processed in chunks of kPermChunk.
constexpr int kPermChunk = 1024;
// Overflow re-routing runs in rounds over blocks of kRerouteTokens tokens; at
// most reroute_rounds(D) rounds before the exact one-wave walk takes over.
constexpr int kRerouteTokens = 256;
inline int reroute_rounds(int D) { return 2 * D + 2; }
// per-block proposal counts are kept expert-major, each expert's row padded to
// a multiple of 4 blocks (16-byte loads)
__host__ __device__ inline int reroute_count_ld(int nb) { return (nb + 3) & ~3; }
// int32 workspace of re-routing: per-block proposal counts (two rounds), the
// re-routed expert and rank per pair, the first pass's offsets, per-token
// state, and one "something was rejected" flag per round
inline int64_t reroute_ws_ints(int64_t T, int k, int E, int D) {
  const int nb = (int)((T + kRerouteTokens - 1) / kRerouteTokens);
  return 2 * (int64_t)reroute_count_ld(nb) * E + 2 * T * k + (E + 1) + T + reroute_rounds(D);
}
struct PermuteLaunch {
  const void* x; const int32_t* topk_idx;
  int32_t* counts; int32_t* offsets; int32_t* dest_row; int32_t* src_token; int32_t* n_dropped;
  void* x_perm;          // null: the rows are not copied (the GEMM gathers them from x)
  int32_t* stats;        // [2E+1] or null
  int32_t* hist;         // workspace [nblocks * E]
  int T, d, E, k, act_bytes;
  int64_t capacity;      // < 0: no limit
  int64_t rows;          // permuted rows provided by the caller
  int fb = 0;            // fallback experts per token after the top-k (topk_idx has k + fb columns)
  int32_t* reroute = nullptr;  // workspace of reroute_ws_ints(T, k, E, fb) (fb > 0 with a limit)
  int32_t* tiles = nullptr;  // or: also write the grouped GEMM's tile lists for tile height
  int tile_bm = 0;           // tile_bm (layout of GemmLaunch::tile_prefix; not with re-routing)
  int32_t* sk_zero = nullptr;  // with tiles: kSkUnits stream-K counters to clear
};
moe_status launch_permute(const PermuteLaunch& a, hipStream_t s);

// load-balancing statistics (balance.hip)
struct RouterStatsLaunch {
  const float* logits; const float* bias; const float* gumbel_u; const int32_t* counts;
  float* prob_mean; float* aux;  // aux may be null
  double* part;                  // workspace of router_stats_ws_bytes(T, E)
  int T, E, score, bias_mode;
  float tau;
};
int64_t router_stats_ws_bytes(int T, int E);
moe_status launch_router_stats(const RouterStatsLaunch& a, hipStream_t s);
moe_status launch_bias_update(const int32_t* counts, float* bias, int E, float decay, float rate, hipStream_t s);

struct CombineLaunch {
  const float* y_perm; const float* y_shared; const int32_t* dest_row; const float* topk_w;
  void* out; int T, d, k, out_dtype;
};
// rows: size of y_perm; destinations outside [0, rows) are ignored
moe_status launch_combine(const CombineLaunch& a, hipStream_t s, int64_t rows);

// Grouped GEMM over experts.  Rows of group g are [offsets[g], offsets[g+1]) of A
// (or [0, single_rows) when offsets == null).  B is [groups][n_b][K] ([out, in]).
struct GemmLaunch {
  const void* A;            // [rows, K] bf16 or f32
  const void* B0;           // gate (gated) or down weights
  const void* B1;           // up weights (gated) or null
  const void* S0;           // B0's scales: fp8 f32 row scales [groups][n_b]; INT4 uint32
  const void* S1;           // group words [groups][n_b][K/128]; else null
  void* out;                // gated: h [rows, F] (bf16 or f32); else y [rows, N] f32
  const int32_t* offsets;   // [groups+1] or null
  int32_t* tile_prefix;     // workspace [2 * (groups+1) + ceil(max_rows/16) + groups]: sanitised
                            // offsets, tile prefix, group of each m-tile (tile_list_ints)
  int groups;
  int single_rows;          // rows when offsets == null
  int64_t max_rows;         // upper bound on rows (grid sizing)
  int K;                    // reduction size
  int N;                    // output columns (F for gated, d for down)
  int w_dtype;              // MOE_F32 / MOE_BF16 / MOE_FP8_E4M3FN / MOE_INT4
  bool gated;
  bool shared;              // the shared expert (names its launches apart)
  const int32_t* gather = nullptr;  // row r of A is A[gather[r]] (A = x, gather = src_token), or
                                    // null for a dense A; only kernels that gather_ok() admits
  int64_t group_rows_max = -1;  // most rows any group can hold (the capacity), or -1: unknown
  bool tiles_ready = false; // tile_prefix already holds this launch's tile lists (same
                            // offsets, groups, max_rows and tile height as a previous launch)
  // stream-K tail of the large-tile kernel: per-unit partial slots (one
  // 256 x 256 f32 tile per CU, at most kSkUnits) and one arrival counter per
  // tail tile (kSkUnits ints; zero between launches: the tile-list writers
  // clear them and the last part of each tile puts its counter back to zero)
  float* sk_part = nullptr;
  int32_t* sk_cnt = nullptr;
};
moe_status launch_grouped_gemm(const GemmLaunch& a, hipStream_t s);
// most stream-K units of one large-tile launch (units run one per CU)
constexpr int kSkUnits = 1024;
// rows per tile of the kernel launch_grouped_gemm picks for `a`
int grouped_gemm_bm(const GemmLaunch& a);
// int32 entries of GemmLaunch::tile_prefix for `groups` groups of at most `max_rows` rows in all
inline int64_t tile_list_ints(int groups, int64_t max_rows) {
  return 2 * (int64_t)(groups + 1) + (max_rows + 15) / 16 + groups;
}
// whether the kernel launch_grouped_gemm picks for `a` can read A through a.gather
// (row byte offsets into A must also fit 32 bits: A_rows * K * 2 < 2^32)
bool gather_ok(const GemmLaunch& a, int64_t a_rows);





}  // namespace moe
