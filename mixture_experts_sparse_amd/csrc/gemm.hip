// Grouped SwiGLU expert GEMMs.
//
// Page "MoE sparse activation: principles and engineering practice"
// (kapook.pages.dev), s4.2 expert fusion: the tokens routed to one expert are
// batched into one large matmul so the matrix cores run dense tiles.  Page
// "GPT-4 has 1.8T parameters but uses 2% per token" (mlqm.cn), s3.3: the
// expert FFN uses SwiGLU; the three-matrix form
//     h = silu(x W_gate^T) * (x W_up^T),   y = h W_down^T
// is computed in two passes:
//   gated pass : B rows = W_gate and W_up of one expert; epilogue forms h
//   down pass  : B rows = W_down of one expert; epilogue writes y in f32
//
// Every group (expert) owns rows [goff[g], goff[g+1]) of A.  A tiny kernel
// sanitises the caller's offsets and builds the tile prefix (m-tiles per
// group); the GEMM is persistent: each block walks tiles L in
// (group, n-tile, m-tile) order, so the m-tiles sharing one weight tile run
// side by side, and consecutive L stay on one XCD (blocks are dispatched to
// the 8 XCDs round-robin, so block b serves XCD b % 8 and the tile range of
// that XCD), where they share its L2.
//
// bf16 / fp8 weights: v_mfma_f32_16x16x32_bf16, block tile 128 x 128, K step
// 64, four waves of 64 x 64, LDS double buffer (one barrier per K step).  fp8
// (OCP e4m3fn) codes are converted exactly to bf16 on their way into LDS; the
// per-output-row scale multiplies the f32 accumulator in the epilogue.
// fp32 weights: a plain LDS-tiled SIMT kernel (the tiny fp32 workload).
#include <algorithm>

#include "grouped.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- tile list
// goff[g] = running max of clamp(offsets[g], 0, max_rows); tiles[g] = ceil(rows/bm);
// tile_prefix = exclusive scan of tiles, then the group of every m-tile.
// groups + 1 <= 512.
__global__ __launch_bounds__(512) void tiles_kernel(const int32_t* __restrict__ offsets, int groups,
                                                    int single_rows, int64_t max_rows, int bm,
                                                    int32_t* __restrict__ goff,
                                                    int32_t* __restrict__ tile_prefix,
                                                    int32_t* __restrict__ sk_zero) {
  __shared__ int o[512];
  if (sk_zero)  // the large-tile GEMM's stream-K counters start at zero
    for (int j = threadIdx.x; j < kSkUnits; j += 512) sk_zero[j] = 0;
  __shared__ int tp[512];
  const int i = threadIdx.x;
  int v = 0;
  if (i <= groups) {
    if (offsets) {
      int64_t x = offsets[i];
      x = x < 0 ? 0 : (x > max_rows ? max_rows : x);
      v = (int)x;
    } else {
      v = (i == 0) ? 0 : single_rows;
    }
  }
  o[i] = (i == 0) ? 0 : v;  // the first group always starts at row 0
  __syncthreads();
  for (int off = 1; off < 512; off <<= 1) {  // prefix max -> monotone offsets
    int w = (i >= off) ? o[i - off] : 0;
    __syncthreads();
    o[i] = max(o[i], w);
    __syncthreads();
  }
  int tiles = (i < groups) ? (o[i + 1] - o[i] + bm - 1) / bm : 0;
  tp[i] = tiles;
  __syncthreads();
  for (int off = 1; off < 512; off <<= 1) {  // inclusive sum scan
    int w = (i >= off) ? tp[i - off] : 0;
    __syncthreads();
    tp[i] += w;
    __syncthreads();
  }
  if (i <= groups) {
    goff[i] = o[i];
    tile_prefix[i] = (i == 0) ? 0 : tp[i - 1];
  }
  // the group of each m-tile (group-major order), after the prefix: map_tile
  // finds a tile's group with one load instead of a search over the prefix
  if (i < groups) {
    int32_t* tile_group = tile_prefix + groups + 1;
    const int first = (i == 0) ? 0 : tp[i - 1];
    for (int m = first; m < tp[i]; ++m) tile_group[m] = i;
  }
}

struct GemmParams {
  const void* A;
  const void* B0;
  const void* B1;
  const float* S0;
  const float* S1;
  void* out;
  const int32_t* goff;
  const int32_t* tp;
  int groups, K, N, n_tiles;
};

// ---------------------------------------------------------------- MFMA kernel
constexpr int MB = 128, NB = 128, KB = 64, LDK = KB + 8;  // LDS row stride (bf16) breaks bank conflicts

template <bool GATED, bool FP8>
__global__ __launch_bounds__(256, 2) void gemm_mfma_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][MB * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][NB * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int K = p.K, N = p.N;
  const int total = p.n_tiles * p.tp[p.groups];
  const int G8 = gridDim.x >> 3, xcd = blockIdx.x & 7, jb = blockIdx.x >> 3;
  const int chunk = (total + 7) >> 3;
  const int lend = min(total, (xcd + 1) * chunk);
  const uint16_t* A = (const uint16_t*)p.A;
  const int ksteps = K / KB;

  for (int L = xcd * chunk + jb; L < lend; L += G8) {
    const TileRef tr = map_tile(L, p.n_tiles, p.groups, MB, p.tp, p.goff);
    const int g = tr.g;

    // ---- per-thread global sources for this tile (offsets in elements of A / bytes of B)
    // thread chunk i covers LDS row (tid + 256 i) / 8 of A (16-byte column (tid & 7))
    const int a_r = tid >> 3, a_c = (tid & 7) * 8;
    const uint16_t* a0 = A + (size_t)(tr.row0 + min(a_r, tr.rows - 1)) * K + a_c;
    const uint16_t* a1 = A + (size_t)(tr.row0 + min(a_r + 32, tr.rows - 1)) * K + a_c;
    const uint16_t* a2 = A + (size_t)(tr.row0 + min(a_r + 64, tr.rows - 1)) * K + a_c;
    const uint16_t* a3 = A + (size_t)(tr.row0 + min(a_r + 96, tr.rows - 1)) * K + a_c;
    // B: bf16 -> 4 chunks (rows tid/8 + 32 i), fp8 -> 2 chunks (rows tid/4 + 64 i)
    constexpr int BRS = FP8 ? 64 : 32;          // row step between a thread's chunks
    const int b_r = FP8 ? (tid >> 2) : (tid >> 3);
    const size_t b_c = FP8 ? (size_t)(tid & 3) * 16 : (size_t)(tid & 7) * 16;  // bytes
    constexpr size_t EB = FP8 ? 1 : 2;
    auto brow = [&](int r) -> const uint8_t* {
      int wrow;
      const void* base;
      if (GATED) {
        const int half = r >> 6, q = r & 63;
        wrow = tr.nt * 64 + half * 32 + (q & 31);
        base = (q < 32) ? p.B0 : p.B1;
      } else {
        wrow = tr.nt * NB + r;
        base = p.B0;
      }
      return (const uint8_t*)base + ((size_t)g * N * K + (size_t)wrow * K) * EB + b_c;
    };
    const uint8_t* b0 = brow(b_r);
    const uint8_t* b1 = brow(b_r + BRS);
    const uint8_t* b2 = FP8 ? nullptr : brow(b_r + 2 * BRS);
    const uint8_t* b3 = FP8 ? nullptr : brow(b_r + 3 * BRS);

    uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
#define MOE_GLOAD(kstep)                                  \
  do {                                                    \
    const size_t ka_ = (size_t)(kstep) * KB;              \
    ra0 = *(const uint4*)(a0 + ka_);                      \
    ra1 = *(const uint4*)(a1 + ka_);                      \
    ra2 = *(const uint4*)(a2 + ka_);                      \
    ra3 = *(const uint4*)(a3 + ka_);                      \
    rb0 = *(const uint4*)(b0 + ka_ * EB);                 \
    rb1 = *(const uint4*)(b1 + ka_ * EB);                 \
    if (!FP8) {                                           \
      rb2 = *(const uint4*)(b2 + ka_ * EB);               \
      rb3 = *(const uint4*)(b3 + ka_ * EB);               \
    }                                                     \
  } while (0)
#define MOE_BSTORE_FP8(buf, reg, row)                                   \
  do {                                                                  \
    uint4 lo_, hi_;                                                     \
    fp8x16_to_bf16x16(reg, lo_, hi_);                                   \
    *(uint4*)&Bs[buf][(row) * LDK + (tid & 3) * 16] = lo_;              \
    *(uint4*)&Bs[buf][(row) * LDK + (tid & 3) * 16 + 8] = hi_;          \
  } while (0)
#define MOE_LSTORE(buf)                                                 \
  do {                                                                  \
    *(uint4*)&As[buf][(a_r) * LDK + a_c] = ra0;                         \
    *(uint4*)&As[buf][(a_r + 32) * LDK + a_c] = ra1;                    \
    *(uint4*)&As[buf][(a_r + 64) * LDK + a_c] = ra2;                    \
    *(uint4*)&As[buf][(a_r + 96) * LDK + a_c] = ra3;                    \
    if (FP8) {                                                          \
      MOE_BSTORE_FP8(buf, rb0, b_r);                                    \
      MOE_BSTORE_FP8(buf, rb1, b_r + 64);                               \
    } else {                                                            \
      *(uint4*)&Bs[buf][(b_r) * LDK + (tid & 7) * 8] = rb0;             \
      *(uint4*)&Bs[buf][(b_r + 32) * LDK + (tid & 7) * 8] = rb1;        \
      *(uint4*)&Bs[buf][(b_r + 64) * LDK + (tid & 7) * 8] = rb2;        \
      *(uint4*)&Bs[buf][(b_r + 96) * LDK + (tid & 7) * 8] = rb3;        \
    }                                                                   \
  } while (0)

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    MOE_GLOAD(0);
    MOE_LSTORE(0);
    __syncthreads();
    for (int ks = 0; ks < ksteps; ++ks) {
      const int buf = ks & 1;
      if (ks + 1 < ksteps) MOE_GLOAD(ks + 1);
#pragma unroll
      for (int kk = 0; kk < KB; kk += 32) {
        bf16x8_t af[4], bfr[4];
        const int koff = kk + (lane >> 4) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          af[i] = *(const bf16x8_t*)&As[buf][(wm * 64 + i * 16 + (lane & 15)) * LDK + koff];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bfr[j] = *(const bf16x8_t*)&Bs[buf][(wn * 64 + j * 16 + (lane & 15)) * LDK + koff];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(af[i], bfr[j], acc[i][j]);
      }
      if (ks + 1 < ksteps) MOE_LSTORE(buf ^ 1);
      __syncthreads();
    }

    // ---- epilogue
    const int col_in = lane & 15;
    const int rquad = (lane >> 4) * 4;
    if (GATED) {
      uint16_t* h = (uint16_t*)p.out;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int f = tr.nt * 64 + wn * 32 + j * 16 + col_in;
        float sg = 1.f, su = 1.f;
        if (FP8) { sg = p.S0[(size_t)g * N + f]; su = p.S1[(size_t)g * N + f]; }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = wm * 64 + i * 16 + rquad + r;
            if (m < tr.rows) {
              const float gv = acc[i][j][r] * sg;
              const float uv = acc[i][j + 2][r] * su;
              h[(size_t)(tr.row0 + m) * N + f] = f32_to_bf16_rne(silu_f32(gv) * uv);
            }
          }
      }
    } else {
      float* y = (float*)p.out;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = tr.nt * NB + wn * 64 + j * 16 + col_in;
        const float sd = FP8 ? p.S0[(size_t)g * N + n] : 1.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = wm * 64 + i * 16 + rquad + r;
            if (m < tr.rows) y[(size_t)(tr.row0 + m) * N + n] = acc[i][j][r] * sd;
          }
      }
    }
  }
}

#undef MOE_GLOAD
#undef MOE_LSTORE
#undef MOE_BSTORE_FP8

// ---------------------------------------------------------------- fp32 SIMT kernel
constexpr int SM = 64, SN = 64, SK = 16;

template <bool GATED>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParams p) {
  __shared__ float As[SK][SM + 4];
  __shared__ float Bs[SK][SN + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int K = p.K, N = p.N;
  const int total = p.n_tiles * p.tp[p.groups];
  const float* A = (const float*)p.A;
  for (int L = blockIdx.x; L < total; L += gridDim.x) {
    const TileRef tr = map_tile(L, p.n_tiles, p.groups, SM, p.tp, p.goff);
    const int g = tr.g;
    // loader: one float4 of A and one of B per thread per K step
    const int lr = tid >> 2, lc = (tid & 3) * 4;
    const float* a_src = A + (size_t)(tr.row0 + min(lr, tr.rows - 1)) * K + lc;
    const float* b_src;
    if (GATED) {
      const int q = lr;  // rows 0..31 gate, 32..63 up
      const float* base = (const float*)((q < 32) ? p.B0 : p.B1);
      b_src = base + (size_t)g * N * K + (size_t)(tr.nt * 32 + (q & 31)) * K + lc;
    } else {
      b_src = (const float*)p.B0 + (size_t)g * N * K + (size_t)(tr.nt * SN + lr) * K + lc;
    }
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[i][c] = 0.f;
    int bcol[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) bcol[c] = GATED ? ((c < 2) ? tx * 2 + c : 32 + tx * 2 + (c - 2)) : tx * 4 + c;
    for (int k0 = 0; k0 < K; k0 += SK) {
      const float4 av = *(const float4*)(a_src + k0);
      const float4 bv = *(const float4*)(b_src + k0);
      As[lc + 0][lr] = av.x; As[lc + 1][lr] = av.y; As[lc + 2][lr] = av.z; As[lc + 3][lr] = av.w;
      Bs[lc + 0][lr] = bv.x; Bs[lc + 1][lr] = bv.y; Bs[lc + 2][lr] = bv.z; Bs[lc + 3][lr] = bv.w;
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < SK; ++kk) {
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
        for (int c = 0; c < 4; ++c) b[c] = Bs[kk][bcol[c]];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[i][c] = fmaf(a[i], b[c], acc[i][c]);
      }
      __syncthreads();
    }
    float* out = (float*)p.out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = ty * 4 + i;
      if (m >= tr.rows) continue;
      float* orow = out + (size_t)(tr.row0 + m) * N;
      if (GATED) {
#pragma unroll
        for (int c = 0; c < 2; ++c) orow[tr.nt * 32 + tx * 2 + c] = silu_f32(acc[i][c]) * acc[i][c + 2];
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) orow[tr.nt * SN + tx * 4 + c] = acc[i][c];
      }
    }
  }
}

}  // namespace

// Which kernel runs a pass: the large-tile bf16 kernel when the output width
// tiles evenly (wave tile 128 x 128, or 128 x 64 for narrower outputs), else the
// 128 x 128 kernel (fp8, and bf16 shapes the large tiles do not divide), else
// the fp32 SIMT kernel.
// Kernel choice per pass (rows per group estimated as max_rows / groups):
//   stream (bm 64 or 32; INT4 always 32): fp8 and INT4 weights, or bf16 groups of
//          fewer than 128 rows --
//          bound by reading the weights, so small tiles and full-line streams;
//          groups of at most 16 rows (decode) take bm 16 with K split over the
//          waves of a block, four times the blocks in flight;
//   big (bm 256): bf16 groups of hundreds of rows -- bound by the matrix cores;
//   128 x 128 kernel: any shape the two do not divide; SIMT kernel for fp32.
static bool stream_shape_ok(const GemmLaunch& a) {
  return a.K % 128 == 0 && (a.gated ? (a.N % 128 == 0) : (a.N % 256 == 0));
}
static int stream_bm(const GemmLaunch& a) {
  if (a.w_dtype == MOE_F32 || !stream_shape_ok(a)) return 0;  // (INT4 shapes always fit: checked with the config)
  const int64_t per_group = ceil_div(a.max_rows, std::max(a.groups, 1));
  if (per_group <= 16) return 16;  // K split over the waves of a block
  if (a.w_dtype == MOE_INT4) return 32;
  if (a.w_dtype == MOE_BF16 && per_group >= 128) return 0;
  return per_group <= 32 ? 32 : 64;
}
static bool use_big(const GemmLaunch& a) {
  if (a.w_dtype != MOE_BF16 || a.K % 64 || stream_bm(a)) return false;
  return a.gated ? (a.N % 128 == 0) : (a.N % 256 == 0);
}

bool gather_ok(const GemmLaunch& a, int64_t a_rows) {
  if (!use_big(a) && !stream_bm(a)) return false;
  return a_rows * (int64_t)a.K * 2 < ((int64_t)1 << 32);
}

int grouped_gemm_bm(const GemmLaunch& a) {
  if (a.w_dtype == MOE_F32) return SM;
  if (use_big(a)) return 256;
  const int sbm = stream_bm(a);
  return sbm ? sbm : MB;
}

moe_status launch_grouped_gemm(const GemmLaunch& a, hipStream_t s) {
  const bool f32 = (a.w_dtype == MOE_F32);
  const bool big = use_big(a);
  const int sbm = stream_bm(a);
  if (a.gather && !big && !sbm) return fail(MOE_ERR_UNSUPPORTED, "row gather needs the large-tile or streaming GEMM");
  if (a.w_dtype == MOE_INT4 && !sbm) return fail(MOE_ERR_UNSUPPORTED, "INT4 weights need K %% 128 == 0 and N %% 256 == 0");
  const int bm = grouped_gemm_bm(a);
  int32_t* goff = a.tile_prefix;
  int32_t* tp = a.tile_prefix + (a.groups + 1);
  moe_status st;
  int tok;
  if (!a.tiles_ready) {
    tok = begin_launch("gemm_tiles", s);
    hipLaunchKernelGGL(tiles_kernel, dim3(1), dim3(512), 0, s, a.offsets, a.groups, a.single_rows,
                       a.max_rows, bm, goff, tp, a.sk_cnt);
    st = end_launch(tok, s);
    if (st != MOE_OK) return st;
  }

  if (big) return launch_gemm_bf16_big(a, goff, tp, s);
  if (sbm == 16) return launch_gemm_ksplit(a, goff, tp, s);
  if (sbm) return launch_gemm_stream(a, goff, tp, sbm, s);
  GemmParams p{a.A, a.B0, a.B1, (const float*)a.S0, (const float*)a.S1, a.out, goff, tp, a.groups, a.K, a.N, 0};
  const int64_t mt_upper = ceil_div(a.max_rows, bm) + a.groups;
  if (f32) {
    p.n_tiles = a.gated ? a.N / 32 : a.N / SN;
    const int64_t upper = mt_upper * p.n_tiles;
    const int grid = (int)std::min<int64_t>(upper, (int64_t)device_cu_count() * 4);
    if (grid <= 0) return MOE_OK;
    tok = begin_launch(a.shared ? (a.gated ? "shared_f32_gate_up" : "shared_f32_down")
                                : (a.gated ? "gemm_f32_gate_up" : "gemm_f32_down"), s);
    if (a.gated) hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3(grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3(grid), dim3(256), 0, s, p);
    return end_launch(tok, s);
  }
  p.n_tiles = a.gated ? a.N / 64 : a.N / NB;
  const int64_t upper = mt_upper * p.n_tiles;
  int64_t grid = std::min<int64_t>(upper, (int64_t)device_cu_count() * 2);
  grid = ceil_div(grid, 8) * 8;  // the XCD mapping wants a multiple of 8
  if (grid <= 0) return MOE_OK;
  const bool fp8 = (a.w_dtype == MOE_FP8_E4M3FN);
  const char* name = a.shared ? (a.gated ? (fp8 ? "shared_gate_up_fp8" : "shared_gate_up_bf16")
                                         : (fp8 ? "shared_down_fp8" : "shared_down_bf16"))
                              : (a.gated ? (fp8 ? "gemm_gate_up_fp8" : "gemm_gate_up_bf16")
                                         : (fp8 ? "gemm_down_fp8" : "gemm_down_bf16"));
  tok = begin_launch(name, s);
  if (a.gated) {
    if (fp8) hipLaunchKernelGGL((gemm_mfma_kernel<true, true>), dim3(grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((gemm_mfma_kernel<true, false>), dim3(grid), dim3(256), 0, s, p);
  } else {
    if (fp8) hipLaunchKernelGGL((gemm_mfma_kernel<false, true>), dim3(grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((gemm_mfma_kernel<false, false>), dim3(grid), dim3(256), 0, s, p);
  }
  return end_launch(tok, s);
}

}  // namespace moe
