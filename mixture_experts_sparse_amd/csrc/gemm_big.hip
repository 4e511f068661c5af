// Grouped bf16 expert GEMM with large tiles for expert groups of hundreds of rows.
//
// Same computation and tile walk as gemm.hip (page "MoE sparse activation:
// principles and engineering practice" (kapook.pages.dev), s4.2 expert fusion;
// page "GPT-4 has 1.8T parameters but uses 2% per token" (mlqm.cn), s3.3
// SwiGLU), organised for gfx950's matrix cores:
//
//  * block tile 256 rows x 256 weight rows; eight waves as 2 (M) x 4 (N), each
//    owning a 128 x 64 output tile (128 f32 accumulators per lane);
//  * K step 64 (128-byte LDS rows: every fetch is a whole cache line), filled
//    by direct global -> LDS loads (global_load_lds_dwordx4: lane i of a load
//    lands at base + 16 i), so the prefetch costs no VGPRs.  The activation
//    tile has two 32 KB stages, the weight tile three: the weights are the
//    HBM-first traffic, so their loads get two K steps to land, the activation
//    rows (shared by eight CUs of an XCD and cache-resident) one.  160 KB in all;
//  * 16-byte chunk c of row r is stored at slot c ^ (r & 7): the 16x16x32
//    fragment reads (row = lane % 16, chunk = lane / 16 (+4)) are then free of
//    bank conflicts.  The swizzle is applied on the load side by choosing
//    which global chunk each lane fetches;
//  * each K step is two 32-wide halves with their own fragment registers: the
//    fragments of one half are read while the MFMAs of the other issue; the
//    single s_barrier of a step sits between the halves, after which the next
//    loads are requested into the stages just consumed;
//  * the eight load instructions of a step are spread one per MFMA row and the
//    twelve fragment reads of a half two per row over the first six rows
//    (scheduling barriers keep that order), so the memory pipeline never gets
//    a burst and the reads have landed before the barrier or the next step
//    waits for them;
//  * the weights are the MFMA's first operand, so a lane's four results are
//    consecutive output columns of one token row: the epilogue stores them
//    straight from the accumulators as 8-byte (h, bf16) or 16-byte (y, f32)
//    vectors, with no LDS staging and no barrier;
//  * persistent: one block per CU walks its XCD's share of the units, so a tile
//    follows the previous one on the same CU with no launch in between
//    (measured at 8 x 1024 rows, 4096 x 14336: gate/up 1517 -> 1447 us);
//  * an expert's rows are spread over its tiles in whole 16-row groups and
//    each wave runs the K loop compiled for its number of live 16-row groups,
//    so padding rows cost loads but almost no MFMAs; experts of more than
//    eight tiles are walked in bands (map_tile_balanced), so the tiles running
//    together on an XCD share their operand tiles in L2.
#include <algorithm>
#include <type_traits>

#include "grouped.h"

namespace moe {
namespace {

#define MOE_GPTR(p) ((const __attribute__((address_space(1))) void*)(p))
#define MOE_LPTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kBK = 64;         // K per stage
constexpr int kBM = 256;        // rows per block tile
constexpr int kRow = kBK * 2;   // bytes per LDS row (bf16)

// s_waitcnt immediates (gfx9 encoding): vmcnt(n) alone, and lgkmcnt(0) alone
constexpr unsigned vmcnt_imm(int n) { return 0x0F70u | (unsigned)(n & 15) | ((unsigned)(n >> 4) << 14); }
constexpr unsigned kLgkm0 = 0xC07Fu;

__device__ __forceinline__ void block_sync() {
  // s_barrier without the memory fence of __syncthreads (which would wait for
  // every load in flight); the empty asm statements keep the compiler from
  // moving memory operations across it.
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct BigParams {
  const void* A;
  const void* B0;
  const void* B1;
  void* out;
  const int32_t* goff;
  const int32_t* tp;
  int groups, K, N, n_tiles;
  const int32_t* gather; // A row r is A[gather[r]], or null
  int G;                 // stream-K: units of the tail round (one per CU), <= kSkUnits
  float* sk_part;        // G partial slots of 64 Ki floats (one per tail unit), or null: no stream-K
  int32_t* sk_cnt;       // arrival counter per tail tile (zero between launches)
};

constexpr int kMinSkSteps = 16;  // K steps of the shortest stream-K fragment

// Waves: 2 along M (128 rows each) x 4 along N (64 weight rows each).
template <bool GATED>
__global__ __launch_bounds__(512, 1) void gemm_bf16_big_kernel(BigParams p) {
  constexpr int WN = 64, WAVES_N = 4, NW = 8;
  constexpr int BNR = WAVES_N * WN;          // 256 weight rows per block
  constexpr int A_BYTES = kBM * kRow;        // 32 KB
  constexpr int B_BYTES = BNR * kRow;        // 32 KB
  constexpr int A_STAGES = 2, B_STAGES = 3;
  constexpr int B_BASE = A_STAGES * A_BYTES; // weight stages follow the activation stages
  constexpr int NJ = WN / 16;                // B fragments per wave
  constexpr int A_INS = A_BYTES / 1024 / NW; // 4 DMA instructions (8 rows each) per wave
  constexpr int B_INS = B_BYTES / 1024 / NW; // 4
  static_assert(A_INS + B_INS == 8, "one load per MFMA row");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[A_STAGES * A_BYTES + B_STAGES * B_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept scalar
  const int wm = w / WAVES_N, wn = w % WAVES_N;
  const int K = p.K, N = p.N;
  const int KS = K / kBK;                              // K steps of a whole tile
  const int n_total = p.n_tiles * p.tp[p.groups];
  // Work units.  Whole tiles (D of them) each make one unit, except that the
  // last R = n_total mod G tiles -- a partial last round -- are cut along K
  // into P parts each (stream-K), P = min(G / R, KS / kMinSkSteps) when that is
  // at least 2: unit D + u is part u % P of tail tile u / P, K steps
  // [KS q / P, KS (q + 1) / P), q = u % P.  Each XCD takes a contiguous share of
  // the whole tiles and then of the tail units, so the parts of one tail tile
  // mostly run on one XCD.
  int R = 0, P = 0;
  if (p.sk_part) {
    R = n_total % p.G;
    P = R ? min(p.G / R, KS / kMinSkSteps) : 0;
    if (P < 2) R = P = 0;
  }
  const int D = n_total - R, NU = R * P;
  const int G8 = gridDim.x >> 3, xcd = blockIdx.x & 7, jb = blockIdx.x >> 3;
  const int dp0 = (int)((int64_t)D * xcd / 8), n_dp = (int)((int64_t)D * (xcd + 1) / 8) - dp0;
  const int sk0 = NU * xcd / 8, n_x = n_dp + NU * (xcd + 1) / 8 - sk0;

  // per-lane constants of the swizzled layout
  const int dma_row = lane >> 3;                  // row inside an 8-row slab
  const int dma_chunk = (lane & 7) ^ dma_row;     // global 16-byte chunk this lane fetches
  const int frow = lane & 15;
  const int kg = lane >> 4;                       // k group of the fragment (8 values each)
  const uint32_t a_frag0 = (uint32_t)((wm * 128 + frow) * kRow + ((kg ^ (frow & 7)) * 16));
  const uint32_t a_frag1 = (uint32_t)((wm * 128 + frow) * kRow + (((kg + 4) ^ (frow & 7)) * 16));
  const uint32_t b_frag0 = (uint32_t)((wn * WN + frow) * kRow + ((kg ^ (frow & 7)) * 16));
  const uint32_t b_frag1 = (uint32_t)((wn * WN + frow) * kRow + (((kg + 4) ^ (frow & 7)) * 16));

  for (int local = jb; local < n_x; local += G8) {
    // the unit: tile L, K steps [kbeg, kbeg + ksteps); u = its tail unit, or -1
    const int u = local < n_dp ? -1 : sk0 + local - n_dp;
    int L, kbeg, ksteps;
    if (u < 0) {
      L = dp0 + local;
      kbeg = 0;
      ksteps = KS;
    } else {
      const int q = u % P;
      L = D + u / P;
      kbeg = KS * q / P;
      ksteps = KS * (q + 1) / P - kbeg;
    }
    const TileRef tr = map_tile_balanced(L, p.n_tiles, p.groups, p.tp, p.goff);
    const int g = tr.g;
    const size_t kofs = (size_t)kbeg * kRow;  // byte offset of the fragment's first K step

    // load sources: wave-uniform bases plus 32-bit per-lane byte offsets
    // rows past the group's end repeat its last row; with a gather map the rows
    // come straight from the token matrix (offsets checked to fit 32 bits)
    const uint8_t* a_base = (const uint8_t*)p.A + (p.gather ? 0 : (size_t)tr.row0 * K * 2) + kofs;
    uint32_t a_off[A_INS];
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
      const int r = min((w * A_INS + i) * 8 + dma_row, tr.rows - 1);
      const uint32_t src = p.gather ? (uint32_t)p.gather[tr.row0 + r] : (uint32_t)r;
      a_off[i] = (src * (uint32_t)K + (uint32_t)(dma_chunk * 8)) * 2u;
    }
    const uint32_t b_off = (uint32_t)((dma_row * K + dma_chunk * 8) * 2);
    const uint8_t* b_base[B_INS];
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
      const int r0 = (w * B_INS + i) * 8;  // first row of this 8-row slab
      int wrow0;
      const void* base;
      if (GATED) {
        // wave slab `half`: WN/2 gate rows then the WN/2 matching up rows
        const int half = r0 / WN, q = r0 % WN;
        wrow0 = tr.nt * (BNR / 2) + half * (WN / 2) + (q % (WN / 2));
        base = (q < WN / 2) ? p.B0 : p.B1;
      } else {
        wrow0 = tr.nt * BNR + r0;
        base = p.B0;
      }
      b_base[i] = (const uint8_t*)base + ((size_t)g * N * K + (size_t)wrow0 * K) * 2 + kofs;
    }
    // load instruction q (0..7) of step ks into that step's stage (activation
    // stage ks % 2, weight stage ks % 3); steps past the last are clamped to it
    // (they refill a stage just consumed, which no later step reads)
    auto load_one = [&](int q, int ks) {
      const uint32_t kb = (uint32_t)min(ks, ksteps - 1) * kRow;
      if (q < A_INS)
        __builtin_amdgcn_global_load_lds(MOE_GPTR(a_base + a_off[q] + kb),
                                         MOE_LPTR(smem + (ks & 1) * A_BYTES + (w * A_INS + q) * 1024), 16, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(MOE_GPTR(b_base[q - A_INS] + b_off + kb),
                                         MOE_LPTR(smem + B_BASE + (ks % 3) * B_BYTES + (w * B_INS + q - A_INS) * 1024),
                                         16, 0, 0);
    };

    f32x4_t acc[8][NJ];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    bf16x8_t X[8 + NJ], Y[8 + NJ];  // fragments of the first / second 32-wide half of a step

    block_sync();  // every wave is done with the previous unit's stages
    // activations of steps 0 and 1, weights of steps 0, 1 and 2 (in this order:
    // loads complete in issue order, so a count of outstanding loads names them)
#pragma unroll
    for (int q = 0; q < 8; ++q) load_one(q, 0);
#pragma unroll
    for (int q = 0; q < 8; ++q) load_one(q, 1);
#pragma unroll
    for (int q = A_INS; q < 8; ++q) load_one(q, 2);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(8 + B_INS));  // step 0 has landed
    block_sync();

    // 16-row groups of this wave's 128 rows that hold rows of the tile: the MFMA
    // rows of the others would only multiply padding
    const int live = min(8, max(0, tr.rows - wm * 128 + 15) / 16);
    // fragment entry e of a half: weights first (every MFMA row needs all of
    // them), then the activation rows
    auto read_frag = [&](bf16x8_t (&F)[8 + NJ], int e, const uint8_t* sa, const uint8_t* sb, uint32_t af,
                         uint32_t bf) {
      if (e < NJ) F[8 + e] = *(const bf16x8_t*)(sb + bf + e * 2048);
      else F[e - NJ] = *(const bf16x8_t*)(sa + af + (e - NJ) * 2048);
    };
    // the K loop for NI live groups (NI = 0: the wave only takes its share of the
    // loads, with the same waits and the same one barrier per step)
    auto k_loop = [&](auto ni) {
      constexpr int NI = decltype(ni)::value;
      if constexpr (NI == 0) {
        for (int ks = 0; ks < ksteps; ++ks) {
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(B_INS));
          block_sync();
#pragma unroll
          for (int i = 0; i < 8; ++i) load_one(i, i < A_INS ? ks + 2 : ks + 3);
        }
      } else {
        constexpr int NE = NJ + NI;                  // fragment reads per half
        constexpr int RPR = (NE + NI - 1) / NI;      // of them per MFMA row
        constexpr int LPR = (8 + NI - 1) / NI;       // load instructions per MFMA row
#pragma unroll
        for (int e = 0; e < NE; ++e) read_frag(X, e, smem, smem + B_BASE, a_frag0, b_frag0);
        // nothing may be pending at the loop head (tile lookups leave scalar loads in
        // flight, which would make the compiler drain the counter there every step)
        __builtin_amdgcn_s_waitcnt(kLgkm0);
        int bs = 0;  // weight stage of step ks (ks % 3)
        for (int ks = 0; ks < ksteps; ++ks) {
          const int bn = bs == 2 ? 0 : bs + 1;
          const uint8_t* sa = smem + (ks & 1) * A_BYTES;
          const uint8_t* sb = smem + B_BASE + bs * B_BYTES;
          const uint8_t* na = smem + ((ks + 1) & 1) * A_BYTES;
          const uint8_t* nb = smem + B_BASE + bn * B_BYTES;
          // first half: MFMAs on X, second-half fragments of this step read alongside
#pragma unroll
          for (int i = 0; i < NI; ++i) {
#pragma unroll
            for (int e = RPR * i; e < RPR * i + RPR && e < NE; ++e) read_frag(Y, e, sa, sb, a_frag1, b_frag1);
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[i][j] = mfma16x16x32(X[8 + j], X[i], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
          }
          // step ks + 1 has landed; only the weights of step ks + 2 may still be in flight
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(B_INS));
          __builtin_amdgcn_s_waitcnt(kLgkm0);  // this wave's reads of step ks are done
          block_sync();
          // second half: MFMAs on Y; the activations of step ks + 2 and the weights of
          // step ks + 3 requested into the stages step ks has released, and the
          // first-half fragments of step ks + 1 read, spread over the MFMA rows
#pragma unroll
          for (int i = 0; i < NI; ++i) {
#pragma unroll
            for (int q = LPR * i; q < LPR * i + LPR && q < 8; ++q) load_one(q, q < A_INS ? ks + 2 : ks + 3);
#pragma unroll
            for (int e = RPR * i; e < RPR * i + RPR && e < NE; ++e) read_frag(X, e, na, nb, a_frag0, b_frag0);
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[i][j] = mfma16x16x32(Y[8 + j], Y[i], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
          }
          __builtin_amdgcn_s_waitcnt(kLgkm0);  // next step's first-half fragments are in
          bs = bn;
        }
      }
    };
    switch (live) {
      case 8: k_loop(std::integral_constant<int, 8>{}); break;
      case 7: k_loop(std::integral_constant<int, 7>{}); break;
      case 6: k_loop(std::integral_constant<int, 6>{}); break;
      case 5: k_loop(std::integral_constant<int, 5>{}); break;
      case 4: k_loop(std::integral_constant<int, 4>{}); break;
      case 3: k_loop(std::integral_constant<int, 3>{}); break;
      case 2: k_loop(std::integral_constant<int, 2>{}); break;
      case 1: k_loop(std::integral_constant<int, 1>{}); break;
      default: k_loop(std::integral_constant<int, 0>{}); break;
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load may land in a stage after this unit

    if (u >= 0) {
      // A part of a tail tile: its partial sums go to the unit's slot with
      // agent-coherent stores; the last part to arrive (counted by one atomic
      // per tile) adds the P parts in part order -- the sum does not depend on
      // which part finishes last -- and runs the epilogue.
      const int ts = u / P;
      const size_t lane_base = (size_t)w * (8 * NJ * 4 * 64) + lane;
      auto slot_at = [&](int unit, int i, int j, int r) {
        return p.sk_part + ((size_t)unit << 16) + lane_base + (size_t)((i * NJ + j) * 4 + r) * 64;
      };
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < live)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              __hip_atomic_store(slot_at(u, i, j, r), acc[i][j][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the stores are done
      block_sync();
      if (tid == 0) {
        const int before = __hip_atomic_fetch_add(p.sk_cnt + ts, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = before == P - 1;
        if (last) __hip_atomic_store(p.sk_cnt + ts, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *(volatile int*)smem = last;
        __builtin_amdgcn_s_waitcnt(kLgkm0);
      }
      block_sync();
      const int last = *(volatile int*)smem;
      if (!last) continue;  // (the next unit starts with a barrier before it touches LDS)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i >= live) continue;
        f32x4_t sum[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) sum[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int q = 0; q < P; ++q) {
          const int uq = ts * P + q;
          if (uq == u) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) sum[j] += acc[i][j];
          } else {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                sum[j][r] += __hip_atomic_load(slot_at(uq, i, j, r), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = sum[j];
      }
    }

    // ---- epilogue, straight from the accumulators (rows past the group's end
    // are not stored).  With the weights as the MFMA's first operand, lane l
    // holds token row m = 16 i + l % 16 and the four consecutive output columns
    // 16 j + 4 (l / 16) + r of it, so every store is one 8- or 16-byte vector.
    const int mrow = lane & 15;
    const int nq = (lane >> 4) * 4;
    if (GATED) {
      // h = silu(gate) * up: fragment j < NJ / 2 holds gate columns, j + NJ / 2 the matching up columns
      uint16_t* h = (uint16_t*)p.out + tr.nt * (BNR / 2) + wn * (WN / 2) + nq;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = wm * 128 + i * 16 + mrow;
        if (i >= live || m >= tr.rows) continue;
        uint16_t* hr = h + (size_t)(tr.row0 + m) * N;
#pragma unroll
        for (int j = 0; j < NJ / 2; ++j) {
          uint32_t hv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) hv[r] = f32_to_bf16_rne(silu_f32(acc[i][j][r]) * acc[i][j + NJ / 2][r]);
          *(uint2*)(hr + j * 16) = make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
        }
      }
    } else {
      float* y = (float*)p.out + tr.nt * BNR + wn * WN + nq;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = wm * 128 + i * 16 + mrow;
        if (i >= live || m >= tr.rows) continue;
        float* yr = y + (size_t)(tr.row0 + m) * N;
#pragma unroll
        for (int j = 0; j < NJ; ++j) *(f32x4_t*)(yr + j * 16) = acc[i][j];
      }
    }
  }
}

}  // namespace

// bf16 grouped GEMM with the large-tile kernel: block tile 256 rows x 256 weight rows,
// 8 waves.  Requires N % (gated ? 128 : 256) == 0 and K % 64 == 0 (per K part);
// goff / tile prefix already built for 256-row tiles.
moe_status launch_gemm_bf16_big(const GemmLaunch& a, const int32_t* goff, const int32_t* tp, hipStream_t s) {
  BigParams p{a.A, a.B0, a.B1, a.out, goff, tp, a.groups, a.K, a.N, 0, a.gather, 0, nullptr, nullptr};
  p.n_tiles = a.gated ? a.N / 128 : a.N / 256;
  // the stream-K tail: at most one unit per CU, each at least kMinSkSteps
  // long; the counters were cleared with the tile lists
  if (a.sk_part && a.sk_cnt) {
    p.G = std::min(device_cu_count(), kSkUnits);
    p.sk_part = a.sk_part;
    p.sk_cnt = a.sk_cnt;
  }
  // persistent: one block per CU (rounded down to the 8 XCDs), each taking its
  // XCD's units in turn, so no block waits for a fresh launch between tiles
  const int64_t upper = (ceil_div(a.max_rows, kBM) + a.groups) * p.n_tiles;
  if (upper <= 0) return MOE_OK;
  const int64_t cu8 = std::max<int64_t>(8, device_cu_count() / 8 * 8);
  const int64_t grid = p.G ? cu8 : std::min<int64_t>(ceil_div(upper, 8) * 8, cu8);
  const char* name = a.shared ? (a.gated ? "shared_gate_up_bf16" : "shared_down_bf16")
                              : (a.gated ? "gemm_gate_up_bf16" : "gemm_down_bf16");
  int tok = begin_launch(name, s);
  if (a.gated) hipLaunchKernelGGL(gemm_bf16_big_kernel<true>, dim3(grid), dim3(512), 0, s, p);
  else hipLaunchKernelGGL(gemm_bf16_big_kernel<false>, dim3(grid), dim3(512), 0, s, p);
  return end_launch(tok, s);
}

}  // namespace moe
