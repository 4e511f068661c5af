// Capacity-limited, order-stable permutation of (token, slot) pairs by expert.
//
// Page "Parameter scale and the truth about sparse activation"
// (deepseek.csdn.net), s3.2: capacity = tokens * k / experts * capacity_factor,
// at least 1; pairs over the limit are marked as overflow (dropped here).
// Page "MoE sparse activation: principles and engineering practice"
// (kapook.pages.dev), s4.2 expert fusion: the tokens of one expert are batched
// into one contiguous block so the expert runs one matmul over them.
//
// Pairs p = t*k + j are split into chunks of kPermChunk.  Three small kernels
// compute the same counting sort a sequential walk over p would:
//   hist : per-chunk per-expert counts (LDS atomics; only counts, no order)
//   scan : per expert, exclusive scan over chunks -> chunk base ranks, counts,
//          kept = min(counts, C), offsets, n_dropped
//   rank : stable in-chunk ranks from wave ballots (lanes with the same expert
//          found bit by bit), then rank = base + in-chunk rank; keep iff < C
// and a fourth kernel copies each token's row to its kept destinations.  No
// atomic decides an order, so the result is deterministic.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void hist_kernel(const int32_t* __restrict__ idx,
                                                        int32_t* __restrict__ hist, int P, int E) {
  __shared__ int h[256];
  for (int e = threadIdx.x; e < E; e += kThreads) h[e] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * kPermChunk;
  const int p1 = min(p0 + kPermChunk, P);
  for (int p = p0 + threadIdx.x; p < p1; p += kThreads) {
    const int e = idx[p];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);  // ids outside [0,E) are ignored
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) hist[(size_t)blockIdx.x * E + e] = h[e];
}

// Single block.  hist[b][e] is overwritten with the number of pairs of expert e
// in chunks before b.
__global__ __launch_bounds__(kThreads) void scan_kernel(int32_t* __restrict__ hist, int nblk, int E,
                                                        int64_t cap, int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ n_dropped,
                                                        int32_t* __restrict__ stats) {
  __shared__ int kept_s[256];
  __shared__ int drop_s[256];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int b = 0; b < nblk; ++b) {
      const int c = hist[(size_t)b * E + e];
      hist[(size_t)b * E + e] = run;
      run += c;
    }
  }
  const int kept = (e < E) ? (int)((cap >= 0 && (int64_t)run > cap) ? cap : run) : 0;
  kept_s[e] = kept;
  drop_s[e] = (e < E) ? run - kept : 0;
  __syncthreads();
  // inclusive Hillis-Steele scan of kept over 256 entries
  for (int off = 1; off < 256; off <<= 1) {
    int v = (e >= off) ? kept_s[e - off] : 0;
    int dv = (e >= off) ? drop_s[e - off] : 0;
    __syncthreads();
    kept_s[e] += v;
    drop_s[e] += dv;
    __syncthreads();
  }
  if (e < E) {
    counts[e] = run;
    offsets[e + 1] = kept_s[e];
    if (stats) { stats[e] = run; stats[E + e] = kept; }
  }
  if (e == 0) {
    offsets[0] = 0;
    n_dropped[0] = drop_s[255];
    if (stats) stats[2 * E] = drop_s[255];
  }
}

__global__ __launch_bounds__(kThreads) void rank_kernel(const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ base,
                                                        const int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ dest_row,
                                                        int32_t* __restrict__ src_token,
                                                        int P, int E, int k, int64_t cap,
                                                        int64_t rows) {
  __shared__ int running[256];
  __shared__ int wcnt[4][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < 256; e += kThreads) {
    running[e] = (e < E) ? base[(size_t)blockIdx.x * E + e] : 0;
    wcnt[0][e] = wcnt[1][e] = wcnt[2][e] = wcnt[3][e] = 0;
  }
  const int n_rows = offsets[E];
  __syncthreads();
  const int p0 = blockIdx.x * kPermChunk;
  const int p1 = min(p0 + kPermChunk, P);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r0 = p0; r0 < p1; r0 += kThreads) {  // uniform trip count in the block
    const int p = r0 + tid;
    const int e_in = (p < p1) ? idx[p] : -1;
    const bool valid = e_in >= 0 && e_in < E;  // ids outside [0,E) are dropped uncounted
    const int e = valid ? e_in : 0;
    if (p < p1 && !valid) dest_row[p] = -1;
    // lanes of this wave with the same expert
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint64_t ones = __ballot(valid && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? ones : ~ones;
    }
    const int before = __popcll(peers & lt_mask);
    if (valid && before == 0) wcnt[wave][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int r = running[e] + before;
      for (int w = 0; w < wave; ++w) r += wcnt[w][e];
      if (cap < 0 || (int64_t)r < cap) {
        const int row = offsets[e] + r;
        dest_row[p] = row;
        src_token[row] = p / k;
      } else {
        dest_row[p] = -1;
      }
    }
    __syncthreads();
    for (int x = tid; x < E; x += kThreads) {
      running[x] += wcnt[0][x] + wcnt[1][x] + wcnt[2][x] + wcnt[3][x];
      wcnt[0][x] = wcnt[1][x] = wcnt[2][x] = wcnt[3][x] = 0;
    }
    __syncthreads();
  }
  // rows past the kept ones carry no token; block b clears rows [p0, p0 + chunk)
  // (rows <= P, so the chunks cover every row; kept rows are written above by
  // whichever block owns the pair, and are < n_rows, so the writes are disjoint)
  for (int64_t r = (int64_t)p0 + tid; r < (int64_t)p0 + kPermChunk && r < rows; r += kThreads)
    if (r >= n_rows) src_token[r] = -1;
}

// One wave per token: the row is read once (16-byte vectors, four per lane in
// flight) and written to every kept destination.
__global__ __launch_bounds__(kThreads) void scatter_kernel(const uint4* __restrict__ x,
                                                           const int32_t* __restrict__ dest_row,
                                                           uint4* __restrict__ x_perm, int T,
                                                           int vec_per_row, int k) {
  constexpr int U = 4;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const uint4* src = x + (size_t)t * vec_per_row;
  const int32_t* dr = dest_row + (size_t)t * k;
  for (int v0 = lane; v0 < vec_per_row; v0 += 64 * U) {
    uint4 val[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = v0 + 64 * u;
      val[u] = (v < vec_per_row) ? src[v] : make_uint4(0, 0, 0, 0);
    }
    for (int j = 0; j < k; ++j) {
      const int row = dr[j];
      if (row < 0) continue;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + 64 * u;
        if (v < vec_per_row) x_perm[(size_t)row * vec_per_row + v] = val[u];
      }
    }
  }
}

__global__ void zero_kernel(int32_t* counts, int32_t* offsets, int32_t* n_dropped, int32_t* stats,
                            int E) {
  for (int e = threadIdx.x; e <= 2 * E; e += blockDim.x) {
    if (e < E) counts[e] = 0;
    if (e <= E) offsets[e] = 0;
    if (stats) stats[e] = 0;
  }
  if (threadIdx.x == 0) n_dropped[0] = 0;
}

}  // namespace

moe_status launch_permute(const PermuteLaunch& a, hipStream_t s) {
  const int P = a.T * a.k;
  const int nblk = (int)ceil_div(P, kPermChunk);
  if (P == 0) {
    // nothing routed: counts, offsets and the drop count are zero
    int tok = begin_launch("permute_zero", s);
    hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(kThreads), 0, s, a.counts, a.offsets, a.n_dropped,
                       a.stats, a.E);
    return end_launch(tok, s);
  }
  int tok = begin_launch("permute_hist", s);
  hipLaunchKernelGGL(hist_kernel, dim3(nblk), dim3(kThreads), 0, s, a.topk_idx, a.hist, P, a.E);
  moe_status st = end_launch(tok, s);
  if (st != MOE_OK) return st;

  tok = begin_launch("permute_scan", s);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kThreads), 0, s, a.hist, nblk, a.E, a.capacity,
                     a.counts, a.offsets, a.n_dropped, a.stats);
  st = end_launch(tok, s);
  if (st != MOE_OK) return st;

  tok = begin_launch("permute_rank", s);
  hipLaunchKernelGGL(rank_kernel, dim3(nblk), dim3(kThreads), 0, s, a.topk_idx, a.hist, a.offsets,
                     a.dest_row, a.src_token, P, a.E, a.k, a.capacity, a.rows);
  st = end_launch(tok, s);
  if (st != MOE_OK) return st;

  if (!a.x_perm) return MOE_OK;
  const int vec_per_row = a.d * a.act_bytes / 16;
  tok = begin_launch("permute_scatter", s);
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)ceil_div(a.T, 4)), dim3(kThreads), 0, s,
                     (const uint4*)a.x, a.dest_row, (uint4*)a.x_perm, a.T, vec_per_row, a.k);
  return end_launch(tok, s);
}

}  // namespace moe
