// Weighted combine of the expert outputs back into token order.
//
// Page "MoE sparse activation: principles and engineering practice"
// (kapook.pages.dev), s3.1: the layer output is the sum over the chosen
// experts of gate weight times expert output.  Page "From sparse MoE to
// conditional memory" (m.nxbn.cn), aggregation layer: weighted combine (the
// residual add is the caller's).  Page "V4 full-stack architecture"
// (kwkr.cn), s2.2: the shared expert every token visits, added with weight 1.
//
//   out[t] = sum_{j: dest_row[t,j] >= 0} w[t,j] * y_perm[dest_row[t,j]]  (+ y_shared[t])
//
// Bandwidth-bound: one wave per token (or, for few tokens, wpt waves per
// token, each taking every wpt-th stretch of the row, so a decode batch still
// has hundreds of waves and each makes one or two round trips), 16-byte vector
// loads of the k source rows (gathered by dest_row), up to four slots' rows in
// flight at once, f32 FMAs in j order, one store of the row.
// When the down projection split its reduction, the partial sums of a row are
// added in part order first, so the result does not depend on scheduling.
#include <type_traits>

#include "common.h"

namespace moe {
namespace {

struct Parts {
  const float4* rest;  // parts 1.. of a partial-sum buffer
  size_t stride4;      // float4s between parts
  int n;               // number of parts (1 = a plain buffer)
};

// value of row r, vector v of a buffer that may be split into partial sums
__device__ __forceinline__ float4 load_parts(const float4* __restrict__ first, const Parts& P, size_t off) {
  float4 a = first[off];
  for (int p = 1; p < P.n; ++p) {
    const float4 b = P.rest[(size_t)(p - 1) * P.stride4 + off];
    a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
  }
  return a;
}

template <bool BF16OUT>
__device__ __forceinline__ void store_out(void* out, size_t off, const float4& acc) {
  if (BF16OUT) {
    uint2 o;
    o.x = (uint32_t)f32_to_bf16_rne(acc.x) | ((uint32_t)f32_to_bf16_rne(acc.y) << 16);
    o.y = (uint32_t)f32_to_bf16_rne(acc.z) | ((uint32_t)f32_to_bf16_rne(acc.w) << 16);
    ((uint2*)out)[off] = o;
  } else {
    ((float4*)out)[off] = acc;
  }
}

// wpt waves per token; wave part of a token handles the trips part, part +
// wpt, ... of its row, each lane U 16-byte vectors per trip.  The rows of JB
// slots are requested together (JB x U loads in flight per lane) and then
// added in slot order, so the sum is the same as one slot at a time.
template <bool BF16OUT, int U, int JB>
__global__ __launch_bounds__(256) void combine_kernel(const float4* __restrict__ y_perm,
                                                      const float4* __restrict__ y_shared,
                                                      const int32_t* __restrict__ dest_row,
                                                      const float* __restrict__ topk_w,
                                                      void* __restrict__ out, int T, int vec_per_row,
                                                      int k, int64_t rows, Parts yp, Parts sp, int wpt) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);  // global wave
  const int t = gw / wpt, part = gw - t * wpt;
  if (t >= T) return;
  const int32_t* dr = dest_row + (size_t)t * k;
  const float* wt = topk_w + (size_t)t * k;
  for (int v0 = part * 64 * U + lane; v0 < vec_per_row; v0 += 64 * U * wpt) {
    float4 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < k; j0 += JB) {
      int row[JB];
      float w[JB];
      float4 y[JB][U];
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        const int j = j0 + jj;
        row[jj] = j < k ? dr[j] : -1;
        if (row[jj] >= rows) row[jj] = -1;  // out of range: ignored like a dropped slot
        w[jj] = row[jj] >= 0 ? wt[j] : 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int v = v0 + 64 * u;
          y[jj][u] = (row[jj] >= 0 && v < vec_per_row)
                         ? load_parts(y_perm, yp, (size_t)row[jj] * vec_per_row + v) : make_float4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        if (row[jj] < 0) continue;  // dropped slots add nothing
#pragma unroll
        for (int u = 0; u < U; ++u) {
          acc[u].x = fmaf(w[jj], y[jj][u].x, acc[u].x);
          acc[u].y = fmaf(w[jj], y[jj][u].y, acc[u].y);
          acc[u].z = fmaf(w[jj], y[jj][u].z, acc[u].z);
          acc[u].w = fmaf(w[jj], y[jj][u].w, acc[u].w);
        }
      }
    }
    if (y_shared) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + 64 * u;
        if (v < vec_per_row) {
          const float4 s = load_parts(y_shared, sp, (size_t)t * vec_per_row + v);
          acc[u].x += s.x; acc[u].y += s.y; acc[u].z += s.z; acc[u].w += s.w;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = v0 + 64 * u;
      if (v < vec_per_row) store_out<BF16OUT>(out, (size_t)t * vec_per_row + v, acc[u]);
    }
  }
}

}  // namespace

moe_status launch_combine(const CombineLaunch& a, hipStream_t s, int64_t rows) {
  if (a.T == 0) return MOE_OK;
  const int vec = a.d / 4;
  // waves per token: enough that a small batch fills the chip (about 512 waves),
  // never more than the row's trips
  const int trips = (int)ceil_div(vec, 64 * 4);
  int wpt = 1;
  while (wpt * 2 <= trips && (int64_t)a.T * wpt * 2 <= 512) wpt *= 2;
  const dim3 grid((unsigned)ceil_div((int64_t)a.T * wpt, 4));
  const Parts yp{(const float4*)a.y_rest, a.y_stride / 4, a.y_split};
  const Parts sp{(const float4*)a.sh_rest, a.sh_stride / 4, a.sh_split};
  int tok = begin_launch("combine", s);
  // slots requested together: four at a time when a token has many, or when a
  // small batch leaves registers to spare (measured: one at a time is faster for
  // k <= 2 at full occupancy, where the extra registers cost waves)
  auto go = [&](auto bf16_tag, auto jb_tag) {
    constexpr bool B = decltype(bf16_tag)::value;
    constexpr int JB = decltype(jb_tag)::value;
    hipLaunchKernelGGL((combine_kernel<B, 4, JB>), grid, dim3(256), 0, s, (const float4*)a.y_perm,
                       (const float4*)a.y_shared, a.dest_row, a.topk_w, a.out, a.T, vec, a.k, rows, yp, sp, wpt);
  };
  using I1 = std::integral_constant<int, 1>;
  using I4 = std::integral_constant<int, 4>;
  const bool one = a.k <= 2 && wpt == 1;
  if (a.out_dtype == MOE_BF16) {
    if (one) go(std::true_type{}, I1{}); else go(std::true_type{}, I4{});
  } else {
    if (one) go(std::false_type{}, I1{}); else go(std::false_type{}, I4{});
  }
  return end_launch(tok, s);
}

}  // namespace moe
