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
// (one, count_rank_kernel, when all pairs fit one chunk) compute the same
// counting sort a sequential walk over p would:
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

// expert of pair p = t k + j; the index matrix has ld >= k columns per token
__device__ __forceinline__ int pair_expert(const int32_t* __restrict__ idx, int p, int k, int ld) {
  return idx[(size_t)(p / k) * ld + (p % k)];
}

// Inclusive sums of v and v2 over the block's 256 threads (four waves, thread
// order): shuffles inside each wave, then the wave totals through `tot` (8 ints
// of LDS).  *ta / *tb get the block totals.  Two barriers in all, where a
// Hillis-Steele scan over LDS takes sixteen.
__device__ __forceinline__ void block_scan256(int& v, int& v2, int* tot, int* ta, int* tb) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int a = __shfl_up(v, off), b = __shfl_up(v2, off);
    if (lane >= off) {
      v += a;
      v2 += b;
    }
  }
  if (lane == 63) {
    tot[w] = v;
    tot[4 + w] = v2;
  }
  __syncthreads();
  int pa = 0, pb = 0;
  for (int i = 0; i < w; ++i) {
    pa += tot[i];
    pb += tot[4 + i];
  }
  *ta = tot[0] + tot[1] + tot[2] + tot[3];
  *tb = tot[4] + tot[5] + tot[6] + tot[7];
  v += pa;
  v2 += pb;
  __syncthreads();  // tot is free again
}

// The grouped GEMM's tile lists (the layout tiles_kernel writes: offsets,
// exclusive prefix of m-tiles per expert, the expert of every m-tile) from the
// final per-expert row counts, by the one block that knows them.  Thread e holds
// expert e's kept rows and exclusive row offset; `scan` is 256 ints of LDS.
__device__ __forceinline__ void write_tile_lists(int e, int kept, int off_excl, int E, int bm, int* tot,
                                                 int32_t* __restrict__ tiles, int32_t* __restrict__ sk_zero) {
  if (sk_zero)  // the large-tile GEMM's stream-K counters start at zero
    for (int i = e; i < kSkUnits; i += 256) sk_zero[i] = 0;
  const int nt = (e < E) ? (kept + bm - 1) / bm : 0;
  int incl = nt, unused = 0, all_nt, all_unused;
  block_scan256(incl, unused, tot, &all_nt, &all_unused);
  int32_t* goff = tiles;
  int32_t* tp = tiles + E + 1;
  int32_t* tile_group = tiles + 2 * (E + 1);
  if (e < E) {
    goff[e] = off_excl;
    tp[e] = incl - nt;
    for (int m = incl - nt; m < incl; ++m) tile_group[m] = e;
  }
  if (e == E - 1) {
    goff[E] = off_excl + kept;
    tp[E] = incl;
  }
}

__global__ __launch_bounds__(kThreads) void hist_kernel(const int32_t* __restrict__ idx,
                                                        int32_t* __restrict__ hist, int P, int E, int k,
                                                        int ld) {
  __shared__ int h[256];
  for (int e = threadIdx.x; e < E; e += kThreads) h[e] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * kPermChunk;
  const int p1 = min(p0 + kPermChunk, P);
  for (int p = p0 + threadIdx.x; p < p1; p += kThreads) {
    const int e = pair_expert(idx, p, k, ld);
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
                                                        int32_t* __restrict__ stats,
                                                        int32_t* __restrict__ tiles, int tile_bm,
                                                        int32_t* __restrict__ sk_zero) {
  __shared__ int tot[8];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    // chunk counts of this expert, sixteen requested at a time, replaced by
    // the exclusive prefix over chunks
    for (int b0 = 0; b0 < nblk; b0 += 16) {
      int c[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) c[u] = b0 + u < nblk ? hist[(size_t)(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (b0 + u < nblk) {
          hist[(size_t)(b0 + u) * E + e] = run;
          run += c[u];
        }
    }
  }
  const int kept = (e < E) ? (int)((cap >= 0 && (int64_t)run > cap) ? cap : run) : 0;
  int incl = kept, dincl = (e < E) ? run - kept : 0, all_kept, all_drop;
  block_scan256(incl, dincl, tot, &all_kept, &all_drop);
  if (e < E) {
    counts[e] = run;
    offsets[e + 1] = incl;
    if (stats) { stats[e] = run; stats[E + e] = kept; }
  }
  if (e == 0) {
    offsets[0] = 0;
    n_dropped[0] = all_drop;
    if (stats) stats[2 * E] = all_drop;
  }
  if (tiles) write_tile_lists(e, kept, incl - kept, E, tile_bm, tot, tiles, sk_zero);
}

// Stable ranks of the pairs [p0, p1) given running[e] = pairs of expert e before
// p0 (LDS, updated as the chunk is walked) and the kept-row offsets `off` (global
// or LDS): rank = running + lanes of earlier waves + earlier lanes of this wave
// with the same expert (found bit by bit from ballots); kept iff rank < cap.
__device__ __forceinline__ void rank_pairs(const int32_t* __restrict__ idx, int p0, int p1, int E, int k, int ld,
                                           int64_t cap, const int32_t* off, int* running, int (*wcnt)[256],
                                           int32_t* __restrict__ dest_row, int32_t* __restrict__ src_token) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r0 = p0; r0 < p1; r0 += kThreads) {  // uniform trip count in the block
    const int p = r0 + tid;
    const int e_in = (p < p1) ? pair_expert(idx, p, k, ld) : -1;
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
        const int row = off[e] + r;
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
}

__global__ __launch_bounds__(kThreads) void rank_kernel(const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ base,
                                                        const int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ dest_row,
                                                        int32_t* __restrict__ src_token,
                                                        int P, int E, int k, int ld, int64_t cap,
                                                        int64_t rows) {
  __shared__ int running[256];
  __shared__ int wcnt[4][256];
  const int tid = threadIdx.x;
  for (int e = tid; e < 256; e += kThreads) {
    running[e] = (e < E) ? base[(size_t)blockIdx.x * E + e] : 0;
    wcnt[0][e] = wcnt[1][e] = wcnt[2][e] = wcnt[3][e] = 0;
  }
  const int n_rows = offsets[E];
  __syncthreads();
  const int p0 = blockIdx.x * kPermChunk;
  const int p1 = min(p0 + kPermChunk, P);
  rank_pairs(idx, p0, p1, E, k, ld, cap, offsets, running, wcnt, dest_row, src_token);
  // rows past the kept ones carry no token; block b clears rows [p0, p0 + chunk)
  // (rows <= P, so the chunks cover every row; kept rows are written above by
  // whichever block owns the pair, and are < n_rows, so the writes are disjoint)
  for (int64_t r = (int64_t)p0 + tid; r < (int64_t)p0 + kPermChunk && r < rows; r += kThreads)
    if (r >= n_rows) src_token[r] = -1;
}

// All pairs in one chunk (P <= kPermChunk, decode-sized batches): the
// histogram, the offsets and the ranks of hist_kernel, scan_kernel and
// rank_kernel in one block, so a small batch pays one launch instead of three.
__global__ __launch_bounds__(kThreads) void count_rank_kernel(const int32_t* __restrict__ idx, int P, int E,
                                                              int k, int ld, int64_t cap, int64_t rows,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ n_dropped,
                                                              int32_t* __restrict__ stats,
                                                              int32_t* __restrict__ dest_row,
                                                              int32_t* __restrict__ src_token,
                                                              int32_t* __restrict__ tiles, int tile_bm,
                                                              int32_t* __restrict__ sk_zero) {
  __shared__ int running[256];
  __shared__ int wcnt[4][256];
  __shared__ int32_t off_s[257];
  __shared__ int32_t idx_s[kPermChunk];  // the pairs' experts, read from memory once
  __shared__ int tot[8];
  const int tid = threadIdx.x;
  running[tid] = 0;
  wcnt[0][tid] = wcnt[1][tid] = wcnt[2][tid] = wcnt[3][tid] = 0;
  for (int p = tid; p < P; p += kThreads) idx_s[p] = pair_expert(idx, p, k, ld);
  __syncthreads();
  for (int p = tid; p < P; p += kThreads) {
    const int e = idx_s[p];
    if (e >= 0 && e < E) atomicAdd(&running[e], 1);  // ids outside [0,E) are ignored
  }
  __syncthreads();
  const int e = tid;
  const int run = (e < E) ? running[e] : 0;
  const int kept = (e < E) ? (int)((cap >= 0 && (int64_t)run > cap) ? cap : run) : 0;
  int incl = kept, dincl = run - kept, all_kept, all_drop;
  block_scan256(incl, dincl, tot, &all_kept, &all_drop);
  if (e < E) {
    counts[e] = run;
    offsets[e + 1] = incl;
    off_s[e + 1] = incl;
    if (stats) { stats[e] = run; stats[E + e] = kept; }
  }
  if (e == 0) {
    offsets[0] = 0;
    off_s[0] = 0;
    n_dropped[0] = all_drop;
    if (stats) stats[2 * E] = all_drop;
  }
  if (tiles) write_tile_lists(e, kept, incl - kept, E, tile_bm, tot, tiles, sk_zero);
  running[e] = 0;  // ranks start at zero in the only chunk
  __syncthreads();
  const int n_rows = off_s[E];
  // the cached experts are laid out [T][k]
  rank_pairs(idx_s, 0, P, E, k, k, cap, off_s, running, wcnt, dest_row, src_token);
  for (int64_t r = tid; r < rows; r += kThreads)
    if (r >= n_rows) src_token[r] = -1;
}

// Overflow re-routing (page "Parameter scale and the truth about sparse
// activation" (deepseek.csdn.net), s3.2 level 2: an overflowed token goes to
// its next-best expert that is not full).  The rule is serial: the dropped
// pairs in (t, j) order, each taking the first of its token's D fallback
// experts that is below capacity and not already serving the token.
//
// Two facts make it parallel.  (1) Within a token, the overflowed slots simply
// take the first m available experts of the list in list order (slot order
// follows list order): an entry skipped by one slot stays unavailable for the
// next.  (2) Every expert ranks the tokens the same way, (t) order; then
// deferred acceptance -- every token proposes to its first m entries not yet
// rejected, each expert holds the proposals ranked below its remaining room and
// rejects the rest, rejected tokens propose again -- ends in exactly the serial
// assignment (with one common priority order the stable assignment is unique
// and is the serial one).  A proposal's rank at expert c is the number of
// earlier tokens proposing c: the proposal counts of the blocks before mine
// plus a popcount over a per-expert bitmap of my block's proposers.
//
// Kernels: rr_init_kernel (per token: overflowed slots m, entries that can never
// be taken -- ids outside [0,E), experts already full after the first pass,
// repeats of an earlier entry -- and the first proposals' per-block counts),
// then up to reroute_rounds(D) launches of rr_round_kernel (a round that follows
// one without rejections returns at once), then reroute_kernel: if some round
// rejected nothing, the last round's ranks are final and it only books the
// rows; otherwise the one-wave walk below computes the assignment itself.
//   out: re_e[p] (fallback expert or -1), re_rank[p] (rank among the expert's
//   re-routed pairs), off_first (the first pass's offsets), offsets (final),
//   stats kept / n_dropped (final)

// a token's state word: bits 0-7 entries rejected (or never available), bits
// 8-15 overflowed slots m
__device__ __forceinline__ int rr_props(int rej, int m) {
  int pm = 0, got = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool take = got < m && !((rej >> i) & 1);
    pm |= take ? (1 << i) : 0;
    got += take ? 1 : 0;
  }
  return pm;
}

__device__ __forceinline__ void rr_list(const int32_t* __restrict__ idx, int ld, int k, int D, int t, int (&f)[8]) {
  const int32_t* row = idx + (size_t)t * ld + k;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = i < D ? row[i] : -1;
}

__device__ __forceinline__ bool rr_over(const int32_t* __restrict__ idx, const int32_t* __restrict__ dest_row,
                                        int ld, int k, int E, int t, int j) {
  const int e = idx[(size_t)t * ld + j];
  return e >= 0 && e < E && dest_row[(size_t)t * k + j] < 0;
}

// out[e] = sum of cnt[e * ld + b] over blocks b < nbk, for every expert e < E
// (per-block proposal counts are stored expert-major, ld a multiple of 4 and
// cnt 16-byte aligned).  Thread e reads its expert's run with 16-byte loads,
// 64 blocks' counts in flight at once: the counts were written by the previous
// launch, possibly through another XCD's L2, so each round trip is long.
__device__ __forceinline__ void rr_expert_sums(const int32_t* __restrict__ cnt, int ld, int nbk, int E, int* out) {
  const int e = threadIdx.x;
  if (e >= E) return;
  const int4* row = reinterpret_cast<const int4*>(cnt + (size_t)e * ld);
  int sum = 0;
  for (int b0 = 0; b0 < nbk; b0 += 64) {
    int4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = (b0 + 4 * u < nbk) ? row[b0 / 4 + u] : make_int4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int b = b0 + 4 * u;
      sum += (b < nbk ? v[u].x : 0) + (b + 1 < nbk ? v[u].y : 0) + (b + 2 < nbk ? v[u].z : 0) +
             (b + 3 < nbk ? v[u].w : 0);
    }
  }
  out[e] = sum;
}

__global__ __launch_bounds__(kRerouteTokens) void rr_init_kernel(const int32_t* __restrict__ idx, int ld, int k,
                                                                 int D, int T, int E, int cap,
                                                                 const int32_t* __restrict__ counts,
                                                                 const int32_t* __restrict__ dest_row,
                                                                 int32_t* __restrict__ state,
                                                                 int32_t* __restrict__ cnt0,
                                                                 int32_t* __restrict__ changed, int R) {
  __shared__ int room[256];
  __shared__ int tot[256];
  const int tid = threadIdx.x;
  room[tid] = tid < E ? cap - min(counts[tid], cap) : 0;
  tot[tid] = 0;
  if (blockIdx.x == 0 && tid < R) changed[tid] = 0;
  __syncthreads();
  const int t = blockIdx.x * kRerouteTokens + tid;
  if (t < T) {
    int m = 0;
    for (int j = 0; j < k; ++j) m += rr_over(idx, dest_row, ld, k, E, t, j) ? 1 : 0;
    int f[8];
    rr_list(idx, ld, k, D, t, f);
    int rej = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = f[i];
      bool never = i >= D || c < 0 || c >= E;
      if (!never) never = room[c] <= 0;
#pragma unroll
      for (int i2 = 0; i2 < i; ++i2) never = never || f[i2] == c;
      rej |= never ? (1 << i) : 0;
    }
    state[t] = rej | (m << 8);
    const int pm = m > 0 ? rr_props(rej, m) : 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((pm >> i) & 1) atomicAdd(&tot[f[i]], 1);
  }
  __syncthreads();
  if (tid < E) cnt0[(size_t)tid * reroute_count_ld(gridDim.x) + blockIdx.x] = tot[tid];
}

// One round of deferred acceptance over every token.  cur: the per-block
// counts of this round's proposals (written by the previous launch); nxt: the
// counts of the next round's.  Every overflowed slot's re_e / re_rank is
// written from this round's proposals: after a round without rejections they
// are final.
__global__ __launch_bounds__(kRerouteTokens) void rr_round_kernel(const int32_t* __restrict__ idx, int ld, int k,
                                                                  int D, int T, int E, int cap,
                                                                  const int32_t* __restrict__ counts,
                                                                  const int32_t* __restrict__ dest_row,
                                                                  int32_t* __restrict__ state,
                                                                  const int32_t* __restrict__ cur,
                                                                  int32_t* __restrict__ nxt,
                                                                  int32_t* __restrict__ changed, int r,
                                                                  int32_t* __restrict__ re_e,
                                                                  int32_t* __restrict__ re_rank) {
  if (r > 0 && changed[r - 1] == 0) return;  // an earlier round settled every token
  constexpr int kWords = kRerouteTokens / 32;
  __shared__ int room[256];
  __shared__ int pre[256];
  __shared__ int tot[256];
  __shared__ uint32_t bits[256 * kWords];  // bit (c, tok): my block's token tok proposes c
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  room[tid] = tid < E ? cap - min(counts[tid], cap) : 0;
  tot[tid] = 0;
  rr_expert_sums(cur, reroute_count_ld(gridDim.x), b, E, pre);  // proposals of the blocks before mine
  for (int w = tid; w < E * kWords; w += kRerouteTokens) bits[w] = 0;
  __syncthreads();
  const int t = b * kRerouteTokens + tid;
  const int st = t < T ? state[t] : 0;
  int rej = st & 0xFF;
  const int m = st >> 8;
  int f[8];
  int pm = 0;
  if (m > 0) {
    rr_list(idx, ld, k, D, t, f);
    pm = rr_props(rej, m);
  }
  const int word = tid >> 5;
  const uint32_t below = (1u << (tid & 31)) - 1u;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if ((pm >> i) & 1) atomicOr(&bits[f[i] * kWords + word], 1u << (tid & 31));
  __syncthreads();
  int g[8];
  bool lost = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    g[i] = 0;
    if ((pm >> i) & 1) {
      const int c = f[i];
      const uint32_t* row = bits + c * kWords;
      int rk = pre[c];
      for (int q = 0; q < word; ++q) rk += __popc(row[q]);
      rk += __popc(row[word] & below);
      g[i] = rk;
      if (rk >= room[c]) {
        rej |= 1 << i;
        lost = true;
      }
    }
  }
  if (m > 0) {
    // the a-th overflowed slot (j order) takes the a-th proposal (list order)
    int j = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((pm >> i) & 1) {
        while (j < k && !rr_over(idx, dest_row, ld, k, E, t, j)) ++j;
        if (j < k) {
          re_e[(size_t)t * k + j] = f[i];
          re_rank[(size_t)t * k + j] = g[i];
          ++j;
        }
      }
    }
    for (; j < k; ++j)
      if (rr_over(idx, dest_row, ld, k, E, t, j)) re_e[(size_t)t * k + j] = -1;
  }
  if (lost) {
    state[t] = rej | (m << 8);
    pm = rr_props(rej, m);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if ((pm >> i) & 1) atomicAdd(&tot[f[i]], 1);
  const int any_lost = __syncthreads_or(lost ? 1 : 0);
  if (tid < E) nxt[(size_t)tid * reroute_count_ld(gridDim.x) + b] = tot[tid];
  if (tid == 0 && any_lost) atomicOr(&changed[r], 1);
}

// The exact walk for inputs that the rounds did not settle: one wave over
// chunks of whole tokens in order, the lanes of a chunk settling among
// themselves by the same deferred acceptance (a lane also loses an expert to
// an earlier lane of its own token); the chunk's winners then use up their
// experts' room before the next chunk starts.
// A chunk's inputs, loaded one chunk ahead so the sequential walk never waits
// on memory: the pair's routed expert, its first-pass row and its token's D
// fallback experts (ids outside [0,E) from a caller count as no candidate).
struct RerouteLane {
  int e, d;
  int f0, f1, f2, f3, f4, f5, f6, f7;  // named, not an array: kept in registers
};

__device__ __forceinline__ RerouteLane load_lane(const int32_t* __restrict__ idx, const int32_t* __restrict__ dest_row,
                                                 int ld, int k, int D, int T, int lanes, int t0, int lane) {
  RerouteLane v;
  const int t = t0 + lane / k, j = lane % k;
  const bool active = lane < lanes && t < T;
  v.e = active ? idx[(size_t)t * ld + j] : -1;
  v.d = active ? dest_row[(size_t)t * k + j] : 0;
  const int32_t* f = idx + (size_t)t * ld + k;
  v.f0 = (active && 0 < D) ? f[0] : -1;
  v.f1 = (active && 1 < D) ? f[1] : -1;
  v.f2 = (active && 2 < D) ? f[2] : -1;
  v.f3 = (active && 3 < D) ? f[3] : -1;
  v.f4 = (active && 4 < D) ? f[4] : -1;
  v.f5 = (active && 5 < D) ? f[5] : -1;
  v.f6 = (active && 6 < D) ? f[6] : -1;
  v.f7 = (active && 7 < D) ? f[7] : -1;
  return v;
}

// drop the first fallback: the list moves up one place (the walk only ever
// advances, so the current candidate is always f0 -- no indexed access)
__device__ __forceinline__ void advance(RerouteLane& v) {
  v.f0 = v.f1; v.f1 = v.f2; v.f2 = v.f3; v.f3 = v.f4;
  v.f4 = v.f5; v.f5 = v.f6; v.f6 = v.f7; v.f7 = -1;
}

__global__ __launch_bounds__(64) void reroute_kernel(const int32_t* __restrict__ idx, int ld, int k, int D,
                                                     int T, int E, int cap, const int32_t* __restrict__ counts,
                                                     const int32_t* __restrict__ dest_row,
                                                     int32_t* __restrict__ re_e, int32_t* __restrict__ re_rank,
                                                     const int32_t* __restrict__ changed, int R,
                                                     int32_t* __restrict__ cnt, int nb) {
  __shared__ int room[256];
  __shared__ int given[256];
  const int lane = threadIdx.x;
  // nothing to do when the rounds settled: some round rejected nothing (the
  // flags of the rounds after it stay zero too)
  bool settled_lane = false;
  for (int r = lane; r < R; r += 64) settled_lane = settled_lane || changed[r] == 0;
  if (__ballot(settled_lane) != 0) return;
  for (int e = lane; e < 256; e += 64) {
    room[e] = e < E ? cap - min(counts[e], cap) : 0;
    given[e] = 0;
  }
  __syncthreads();
  const int tpc = 64 / k;      // whole tokens per chunk
  const int lanes = tpc * k;
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const uint64_t tok = (k == 64 ? ~0ull : ((1ull << k) - 1)) << ((lane / k) * k);  // my token's lanes
  RerouteLane nxt = load_lane(idx, dest_row, ld, k, D, T, lanes, 0, lane);
  for (int t0 = 0; t0 < T; t0 += tpc) {
    const RerouteLane cur_in = nxt;
    if (t0 + tpc < T) nxt = load_lane(idx, dest_row, ld, k, D, T, lanes, t0 + tpc, lane);
    const int t = t0 + lane / k, j = lane % k;
    const bool active = lane < lanes && t < T;
    const int p = t * k + j;
    const bool over = active && cur_in.e >= 0 && cur_in.e < E && cur_in.d < 0;
    if (active) re_e[p] = -1;
    if (__ballot(over) == 0) continue;
    RerouteLane fl = cur_in;
    int ptr = 0, cur = -1;
    uint64_t same = 0;  // lanes proposing my expert in the last round
    // every round a lane either keeps its expert or moves on down its list, and
    // a list has D entries: the loop ends after at most lanes * D + 1 rounds
    for (;;) {
      // next candidate; an expert without room at the chunk's start cannot take
      // the lane (room only shrinks within the chunk), so it is skipped at once
      while (over && cur < 0 && ptr < D) {
        const int cand = fl.f0;
        if (cand >= 0 && cand < E && room[cand] > 0) {
          cur = cand;
        } else {
          ++ptr;
          advance(fl);
        }
      }
      const bool prop = over && cur >= 0;
      const int c = prop ? cur : 0;
      same = __ballot(prop);
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const uint64_t ones = __ballot(prop && ((c >> b) & 1));
        same &= ((c >> b) & 1) ? ones : ~ones;
      }
      const bool dup = prop && (same & tok & lt) != 0;  // an earlier slot of my token has it
      const bool hold = prop && !dup;
      const uint64_t holders = same & __ballot(hold);   // lanes keeping the same expert
      const bool lose = dup || (hold && __popcll(holders & lt) >= room[c]);
      if (__ballot(lose) == 0) break;
      if (lose) {
        cur = -1;
        ++ptr;
        advance(fl);
      }
    }
    // commit the chunk (the last round rejected nobody, so every proposing lane
    // won and `same` is the set of winners of my expert): winners take their
    // rank among the expert's re-routed pairs; the last one books the room
    const bool won = over && cur >= 0;
    const int c = won ? cur : 0;
    const uint64_t peers = won ? same : 0ull;
    const int r = __popcll(peers & lt), h = __popcll(peers);
    if (won) {
      re_e[p] = c;
      re_rank[p] = given[c] + r;
    }
    __syncthreads();
    if (won && r == h - 1) {
      given[c] += h;
      room[c] -= h;
    }
    __syncthreads();
  }
  // the rows given to each expert, where rr_finish_kernel sums them (the first
  // block's column of the per-block counts, the other columns zero)
  for (int e = lane; e < E; e += 64)
    for (int b = 0; b < nb; ++b) cnt[(size_t)e * reroute_count_ld(nb) + b] = b == 0 ? given[e] : 0;
}

// Books the rows: kept = the first pass's rows + the re-routed pairs given to
// each expert, their exclusive scan (the final offsets; the first pass's are
// kept for the relocation), the pairs left dropped and the kept statistics.
__global__ __launch_bounds__(256) void rr_finish_kernel(int E, int cap, const int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ off_first,
                                                        const int32_t* __restrict__ cnt, int nb,
                                                        int32_t* __restrict__ n_dropped,
                                                        int32_t* __restrict__ stats) {
  __shared__ int given[256];
  __shared__ int kept_s[256];
  __shared__ int req_s[256];
  const int e = threadIdx.x;
  rr_expert_sums(cnt, reroute_count_ld(nb), nb, E, given);
  const int first = e < E ? offsets[e] : 0;
  const int first_end = e == 0 ? offsets[E] : 0;
  __syncthreads();
  const int kept = e < E ? min(counts[e], cap) + given[e] : 0;
  kept_s[e] = kept;
  req_s[e] = e < E ? counts[e] : 0;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {  // inclusive sum scans
    const int v = e >= off ? kept_s[e - off] : 0;
    const int q = e >= off ? req_s[e - off] : 0;
    __syncthreads();
    kept_s[e] += v;
    req_s[e] += q;
    __syncthreads();
  }
  if (e < E) off_first[e] = first;
  if (e == 0) off_first[E] = first_end;
  if (e < E) {
    offsets[e] = kept_s[e] - kept;
    if (stats) stats[E + e] = kept;
  }
  if (e == 255) {
    offsets[E] = kept_s[255];
    n_dropped[0] = req_s[255] - kept_s[255];
    if (stats) stats[2 * E] = req_s[255] - kept_s[255];
  }
}

// Moves every pair to its final row once the re-routed pairs have been placed:
// first-pass pairs keep their rank within the expert, re-routed pairs follow
// the expert's first-pass rows.
__global__ __launch_bounds__(kThreads) void relocate_kernel(const int32_t* __restrict__ idx, int ld, int k, int E,
                                                            int cap, const int32_t* __restrict__ counts,
                                                            const int32_t* __restrict__ off_first,
                                                            const int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ dest_row,
                                                            const int32_t* __restrict__ re_e,
                                                            const int32_t* __restrict__ re_rank,
                                                            int32_t* __restrict__ src_token, int P) {
  const int p = blockIdx.x * kThreads + threadIdx.x;
  if (p >= P) return;
  const int e = pair_expert(idx, p, k, ld);
  if (e < 0 || e >= E) return;  // ignored ids stay -1
  const int d = dest_row[p];
  int row = -1;
  if (d >= 0) {
    row = offsets[e] + (d - off_first[e]);
  } else {
    const int c = re_e[p];
    if (c >= 0) row = offsets[c] + min(counts[c], cap) + re_rank[p];
  }
  dest_row[p] = row;
  if (row >= 0) src_token[row] = p / k;
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
  const int ld = a.k + a.fb;
  // tile lists for the GEMM when the first pass's rows are final (no re-routing)
  int32_t* tiles = (a.tiles && a.tile_bm > 0 && !(a.fb > 0 && a.capacity >= 0)) ? a.tiles : nullptr;
  int tok;
  moe_status st;
  if (nblk == 1) {
    tok = begin_launch("permute_count_rank", s);
    hipLaunchKernelGGL(count_rank_kernel, dim3(1), dim3(kThreads), 0, s, a.topk_idx, P, a.E, a.k, ld, a.capacity,
                       a.rows, a.counts, a.offsets, a.n_dropped, a.stats, a.dest_row, a.src_token, tiles,
                       a.tile_bm, a.sk_zero);
    st = end_launch(tok, s);
    if (st != MOE_OK) return st;
  } else {
    tok = begin_launch("permute_hist", s);
    hipLaunchKernelGGL(hist_kernel, dim3(nblk), dim3(kThreads), 0, s, a.topk_idx, a.hist, P, a.E, a.k, ld);
    st = end_launch(tok, s);
    if (st != MOE_OK) return st;

    tok = begin_launch("permute_scan", s);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kThreads), 0, s, a.hist, nblk, a.E, a.capacity,
                       a.counts, a.offsets, a.n_dropped, a.stats, tiles, a.tile_bm, a.sk_zero);
    st = end_launch(tok, s);
    if (st != MOE_OK) return st;

    tok = begin_launch("permute_rank", s);
    hipLaunchKernelGGL(rank_kernel, dim3(nblk), dim3(kThreads), 0, s, a.topk_idx, a.hist, a.offsets,
                       a.dest_row, a.src_token, P, a.E, a.k, ld, a.capacity, a.rows);
    st = end_launch(tok, s);
    if (st != MOE_OK) return st;
  }

  if (a.fb > 0 && a.capacity >= 0) {
    const int nb = (int)ceil_div(a.T, kRerouteTokens);
    const size_t cnt_ints = (size_t)reroute_count_ld(nb) * a.E;  // one round's counts
    int32_t* cnt = a.reroute;  // 16-byte aligned: first in the workspace
    int32_t* re_e = cnt + 2 * cnt_ints;
    int32_t* re_rank = re_e + P;
    int32_t* off_first = re_rank + P;
    int32_t* state = off_first + a.E + 1;
    int32_t* changed = state + a.T;
    const int R = reroute_rounds(a.fb);
    const int cap = (int)a.capacity;
    tok = begin_launch("permute_reroute_init", s);
    hipLaunchKernelGGL(rr_init_kernel, dim3(nb), dim3(kRerouteTokens), 0, s, a.topk_idx, ld, a.k, a.fb, a.T, a.E,
                       cap, a.counts, a.dest_row, state, cnt, changed, R);
    st = end_launch(tok, s);
    if (st != MOE_OK) return st;
    for (int r = 0; r < R; ++r) {
      tok = begin_launch("permute_reroute_round", s);
      hipLaunchKernelGGL(rr_round_kernel, dim3(nb), dim3(kRerouteTokens), 0, s, a.topk_idx, ld, a.k, a.fb, a.T,
                         a.E, cap, a.counts, a.dest_row, state, cnt + (r & 1) * cnt_ints,
                         cnt + ((r + 1) & 1) * cnt_ints, changed, r, re_e, re_rank);
      st = end_launch(tok, s);
      if (st != MOE_OK) return st;
    }
    tok = begin_launch("permute_reroute_walk", s);
    hipLaunchKernelGGL(reroute_kernel, dim3(1), dim3(64), 0, s, a.topk_idx, ld, a.k, a.fb, a.T, a.E, cap,
                       a.counts, a.dest_row, re_e, re_rank, changed, R, cnt, nb);
    st = end_launch(tok, s);
    if (st != MOE_OK) return st;
    tok = begin_launch("permute_reroute_finish", s);
    hipLaunchKernelGGL(rr_finish_kernel, dim3(1), dim3(256), 0, s, a.E, cap, a.counts, a.offsets, off_first, cnt, nb,
                       a.n_dropped, a.stats);
    st = end_launch(tok, s);
    if (st != MOE_OK) return st;
    tok = begin_launch("permute_relocate", s);
    hipLaunchKernelGGL(relocate_kernel, dim3((unsigned)ceil_div(P, kThreads)), dim3(kThreads), 0, s, a.topk_idx,
                       ld, a.k, a.E, (int)a.capacity, a.counts, off_first, a.offsets, a.dest_row, re_e, re_rank,
                       a.src_token, P);
    st = end_launch(tok, s);
    if (st != MOE_OK) return st;
  }

  if (!a.x_perm) return MOE_OK;
  const int vec_per_row = a.d * a.act_bytes / 16;
  tok = begin_launch("permute_scatter", s);
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)ceil_div(a.T, 4)), dim3(kThreads), 0, s,
                     (const uint4*)a.x, a.dest_row, (uint4*)a.x_perm, a.T, vec_per_row, a.k);
  return end_launch(tok, s);
}

}  // namespace moe
