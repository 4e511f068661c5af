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
// loads of the k source rows (gathered by dest_row), the rows of one or two
// slots in flight at once, f32 FMAs in j order, one store of the row.
// Expert rows are read and output rows written once: both go through
// non-temporal accesses, which keep them from displacing cache lines other
// data will use (measured 482 -> 444 us at 8192 tokens x 8 slots x 7168; two
// slots of eight vectors per lane instead of four of four: 435 us).
#include <type_traits>

#include "common.h"

namespace moe {
namespace {

// vector off of a row-major f32 buffer read once (non-temporal)
__device__ __forceinline__ float4 load_once(const float4* __restrict__ buf, size_t off) {
  const f32x4_t v = __builtin_nontemporal_load((const f32x4_t*)buf + off);
  return make_float4(v[0], v[1], v[2], v[3]);
}

template <bool BF16OUT>
__device__ __forceinline__ void store_out(void* out, size_t off, const float4& acc) {
  if (BF16OUT) {
    uint2 o;
    o.x = (uint32_t)f32_to_bf16_rne(acc.x) | ((uint32_t)f32_to_bf16_rne(acc.y) << 16);
    o.y = (uint32_t)f32_to_bf16_rne(acc.z) | ((uint32_t)f32_to_bf16_rne(acc.w) << 16);
    ((uint2*)out)[off] = o;
  } else {
    const f32x4_t v = {acc.x, acc.y, acc.z, acc.w};
    __builtin_nontemporal_store(v, (f32x4_t*)out + off);
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
                                                      int k, int64_t rows, int wpt) {
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
                         ? load_once(y_perm, (size_t)row[jj] * vec_per_row + v) : make_float4(0, 0, 0, 0);
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
          const float4 s = load_once(y_shared, (size_t)t * vec_per_row + v);
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
  // slots requested together: two slots of eight vectors per lane; with few
  // tokens, four slots of four vectors (measured at 16384 tokens x 2 slots x
  // 4096, 78 % of the slots dropped: 81.8 -> 76.9 us against one slot of four)
  const bool few = (int64_t)a.T * 2 <= 512;
  const int U = few ? 4 : 8;
  // waves per token: enough that a small batch fills the chip (about 512 waves),
  // never more than the row's trips
  const int trips = (int)ceil_div(vec, 64 * U);
  int wpt = 1;
  while (wpt * 2 <= trips && (int64_t)a.T * wpt * 2 <= 512) wpt *= 2;
  const dim3 grid((unsigned)ceil_div((int64_t)a.T * wpt, 4));
  int tok = begin_launch("combine", s);
  auto go = [&](auto bf16_tag, auto u_tag, auto jb_tag) {
    constexpr bool B = decltype(bf16_tag)::value;
    hipLaunchKernelGGL((combine_kernel<B, decltype(u_tag)::value, decltype(jb_tag)::value>), grid, dim3(256), 0, s,
                       (const float4*)a.y_perm, (const float4*)a.y_shared, a.dest_row, a.topk_w, a.out, a.T, vec,
                       a.k, rows, wpt);
  };
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  using I8 = std::integral_constant<int, 8>;
  auto pick = [&](auto bf16_tag) {
    if (few) go(bf16_tag, I4{}, I4{});
    else go(bf16_tag, I8{}, I2{});
  };
  if (a.out_dtype == MOE_BF16) pick(std::true_type{});
  else pick(std::false_type{});
  return end_launch(tok, s);
}

}  // namespace moe
