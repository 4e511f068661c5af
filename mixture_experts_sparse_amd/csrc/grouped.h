// Tile walk shared by the grouped GEMM kernels.
#pragma once

#include "common.h"

namespace moe {

struct TileRef {
  int g, nt, row0, rows;
};

// Map a linear tile index L (ordered group-major, then n-tile, then m-tile) to
// (group, n-tile, first row, valid rows).  tp = exclusive prefix of m-tiles per
// group followed by the group of each m-tile, goff = sanitised row offsets; all
// built by tiles_kernel.  Group g's tiles are L in [tp[g], tp[g+1]) * n_tiles,
// so L / n_tiles is one of g's m-tile slots and the table names g directly.
__device__ __forceinline__ TileRef map_tile(int L, int n_tiles, int groups, int bm,
                                            const int32_t* __restrict__ tp,
                                            const int32_t* __restrict__ goff) {
  const int g = tp[groups + 1 + L / n_tiles];
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

// The same walk with the group's rows spread evenly over its m-tiles in whole
// 16-row MFMA groups: a group of c rows holds G = ceil(c / 16) such groups, and
// of its mt = ceil(c / bm) tiles, tile mi takes groups [G mi / mt, G (mi + 1) / mt)
// (rows past c cut off).  Tile heights then differ by at most 16 rows, no tile
// is a sliver of a few rows (a sliver costs nearly a whole tile's loads), and
// only the group's last 16-row group can hold padding rows.  G >= mt, so no
// tile is empty, and G <= 16 mt keeps every tile within bm = 256 rows.
//
// Order: a group of more than kBand m-tiles is cut into nb = ceil(mt / kBand)
// bands of about equal height (band b = m-tiles [mt b / nb, mt (b + 1) / nb)),
// walked one after the other, each n-tile by n-tile with its m-tiles
// consecutive.  Tiles that run at the same time on an XCD then share about
// kBand activation tiles and a few weight tiles -- instead of one weight tile
// and one activation tile per tile when a group has dozens of m-tiles -- and
// the loads that miss L2 drop accordingly.  With mt <= kBand (one band) the
// walk is the plain n-tile-major one.
constexpr int kBand = 8;

__device__ __forceinline__ TileRef map_tile_balanced(int L, int n_tiles, int groups,
                                                     const int32_t* __restrict__ tp,
                                                     const int32_t* __restrict__ goff) {
  const int g = tp[groups + 1 + L / n_tiles];
  const int mt = tp[g + 1] - tp[g];
  const int local = L - tp[g] * n_tiles;
  // the band holding m-tile row local / n_tiles (bands start at m-tile mt b / nb)
  const int nb = (mt + kBand - 1) / kBand;
  const int r = local / n_tiles;
  int b = r * nb / mt;
  if (mt * (b + 1) / nb <= r) ++b;
  const int m0 = mt * b / nb, h = mt * (b + 1) / nb - m0;
  const int rem = local - m0 * n_tiles;
  const int nt = rem / h, mi = m0 + rem % h;
  const int c = goff[g + 1] - goff[g];
  const int G = (c + 15) >> 4;
  const int a = (int)(((int64_t)G * mi) / mt) * 16, e = min(c, (int)(((int64_t)G * (mi + 1)) / mt) * 16);
  TileRef t;
  t.g = g;
  t.nt = nt;
  t.row0 = goff[g] + a;
  t.rows = e - a;
  return t;
}

// bf16 large-tile grouped GEMM (gemm_big.hip): block tile 256 x 256, 8 waves of 128 x 64
moe_status launch_gemm_bf16_big(const GemmLaunch& a, const int32_t* goff, const int32_t* tp, hipStream_t s);

// weight-streaming grouped GEMM for groups of few rows (gemm_stream.hip): bf16 or
// fp8 weights, bm = 32 or 64 rows per tile, 256 weight rows per block
moe_status launch_gemm_stream(const GemmLaunch& a, const int32_t* goff, const int32_t* tp, int bm, hipStream_t s);

// weight-streaming grouped GEMM for groups of at most 16 rows (gemm_ksplit.hip):
// 16-row tiles, the block's four waves split K
moe_status launch_gemm_ksplit(const GemmLaunch& a, const int32_t* goff, const int32_t* tp, hipStream_t s);

}  // namespace moe
