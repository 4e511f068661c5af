// Tile walk shared by the grouped GEMM kernels.
#pragma once

#include "common.h"

namespace moe {

struct TileRef {
  int g, nt, row0, rows;
};

// Map a linear tile index L (ordered group-major, then n-tile, then m-tile) to
// (group, n-tile, first row, valid rows).  tp = exclusive prefix of m-tiles per
// group, goff = sanitised row offsets; both built by tiles_kernel.
__device__ __forceinline__ TileRef map_tile(int L, int n_tiles, int groups, int bm,
                                            const int32_t* __restrict__ tp,
                                            const int32_t* __restrict__ goff) {
  int lo = 0, hi = groups;  // largest g with n_tiles * tp[g] <= L
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)tp[mid] * n_tiles <= L) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int mt = tp[g + 1] - tp[g];
  const int local = L - tp[g] * n_tiles;
  const int nt = local / mt, mi = local % mt;
  TileRef r;
  r.g = g;
  r.nt = nt;
  r.row0 = goff[g] + mi * bm;
  r.rows = min(bm, goff[g + 1] - r.row0);
  return r;
}

// bf16 large-tile grouped GEMM (gemm_big.hip): block tile 256 x 256, 8 waves of 128 x 64
moe_status launch_gemm_bf16_big(const GemmLaunch& a, const int32_t* goff, const int32_t* tp, hipStream_t s);

// weight-streaming grouped GEMM for groups of few rows (gemm_stream.hip): bf16 or
// fp8 weights, bm = 32 or 64 rows per tile, 256 weight rows per block
moe_status launch_gemm_stream(const GemmLaunch& a, const int32_t* goff, const int32_t* tp, int bm, hipStream_t s);

}  // namespace moe
