// Grouped expert GEMM for expert groups of few rows: streams the weights.
//
// Same computation and tile walk as gemm.hip (page "MoE sparse activation:
// principles and engineering practice" (kapook.pages.dev), s4.2 expert fusion;
// page "GPT-4 has 1.8T parameters but uses 2% per token" (mlqm.cn), s3.3
// SwiGLU).  When an expert holds tens of rows (capacity-limited or decode
// batches) the pass is bound by reading the weights, so the kernel is built
// around streaming them once at full bandwidth:
//
//  * block = 4 waves x 64 weight rows (256 per block), tile = BM = 16 MF rows
//    of the expert (MF = 2 or 4) -- small tiles waste little MFMA work;
//  * each wave loads its own weight rows straight into registers, 128 k per
//    step: one full 128-byte line per fp8 row (256 bytes per bf16 row), fetched
//    three steps ahead for fp8 (a ring of four register sets) and one step ahead
//    for bf16 -- enough bytes in flight to cover the memory latency at full
//    bandwidth; fp8 (OCP e4m3fn) codes become bf16 in registers
//    (v_cvt_scalef32_pk_bf16_fp8, exact) and row scales multiply the f32
//    accumulators in the epilogue;
//  * the BM activation rows of a step are shared through LDS: three stages
//    filled by direct global -> LDS loads two steps ahead, 16-byte chunk c of
//    row r at slot c ^ (r & 15) so the fragment reads are conflict-free;
//  * lane group g (lane / 16) holds k = 32 g + 8 s .. + 7 in sub-step s of a
//    step, for both operands, so each lane's weight bytes are contiguous.
//
// Group-wise INT4 weights (page "MoE sparse activation: principles and
// engineering practice", s4.2 quantisation: 128 weights per group, each group
// with its own scale and zero point; w = scale * (q - zero)) take a kernel of
// their own with the same activation stages and 32-row tiles (the registers do
// not hold a deeper prefetch ring beside 64-row tiles).  One K step is exactly
// one group, so a lane's 32 codes of a step are one 16-byte load and every
// weight row contributes one 32-bit group word (fp16 scale | zero << 16) per
// step.  A code q becomes the bf16 number 128 + q by bit operations alone
// (0x4300 | q: exponent 2^7, q in the mantissa -- exact), the step's products
// are summed on the MFMA into a per-step accumulator t, one more MFMA against
// a fragment of ones gives the row sums of the activations, and
//     acc += scale * (t - (128 + zero) * rowsum)
// applies the group's parameters once per step and output element.
#include <algorithm>
#include <type_traits>

#include "grouped.h"

namespace moe {
namespace {

#define MOE_GPTR(p) ((const __attribute__((address_space(1))) void*)(p))
#define MOE_LPTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kKS = 128;   // k per step
constexpr int kNST = 3;    // activation stages in LDS

constexpr unsigned vmcnt_imm(int n) { return 0x0F70u | (unsigned)(n & 15) | ((unsigned)(n >> 4) << 14); }
constexpr unsigned kLgkm0 = 0xC07Fu;  // lgkmcnt(0) alone

__device__ __forceinline__ void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Keeps the compiler from reordering memory operations across this point: the
// waits count loads in flight newest first, so load groups must issue in the
// order written.
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

// Steps of the main loop vs the steps after it.  A step's wait counts the loads
// issued behind the ones it needs: the next step's activations and, in the main
// loop, a full group of weight prefetches.  Past the main loop those prefetches
// feed no step, the compiler removes them, and the count must leave them out.
constexpr std::integral_constant<bool, false> kBody{};
constexpr std::integral_constant<bool, true> kTailStep{};

struct StreamParams {
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

// 8 bf16 for sub-step s from a lane's raw weight registers
template <bool FP8>
__device__ __forceinline__ bf16x8_t b_frag(const uint4* raw, int s) {
  if (FP8) {
    // raw[0..1]: 32 fp8 codes (k = 32 g .. 32 g + 31); sub-step s uses bytes 8 s .. 8 s + 7
    const uint4 q = raw[s >> 1];
    const uint32_t lo = (s & 1) ? q.z : q.x, hi = (s & 1) ? q.w : q.y;
    uint4 o;
    o.x = fp8x2_to_bf16x2<false>(lo);
    o.y = fp8x2_to_bf16x2<true>(lo);
    o.z = fp8x2_to_bf16x2<false>(hi);
    o.w = fp8x2_to_bf16x2<true>(hi);
    return __builtin_bit_cast(bf16x8_t, o);
  } else {
    // raw[0..3]: 32 bf16 (k = 32 g .. 32 g + 31); sub-step s uses raw[s]
    return __builtin_bit_cast(bf16x8_t, raw[s]);
  }
}

template <bool GATED, bool FP8, int MF>
__global__ __launch_bounds__(256, 2) void gemm_stream_kernel(StreamParams p) {
  constexpr int BM = 16 * MF;
  constexpr int NF = 4;                    // n-fragments (16 weight rows) per wave
  constexpr int AROW = kKS * 2;            // 256 bytes per activation row
  constexpr int ASTAGE = BM * AROW;
  constexpr int A_INS = BM / 16;           // 1 KB (4 rows) DMA instructions per wave per step
  constexpr int RAW = FP8 ? 2 : 4;         // 16-byte weight registers per n-fragment per step
  __shared__ __attribute__((aligned(1024))) uint8_t As[kNST * ASTAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = p.K, N = p.N, ksteps = K / kKS;
  const int total = p.n_tiles * p.tp[p.groups];
  const int G8 = gridDim.x >> 3, xcd = blockIdx.x & 7, jb = blockIdx.x >> 3;
  const int chunk = (total + 7) >> 3;
  const int lend = min(total, (xcd + 1) * chunk);
  const int g4 = lane >> 4, r16 = lane & 15;
  constexpr size_t EB = FP8 ? 1 : 2;

  // activation DMA: instruction i of wave w covers rows 4 (w A_INS + i) .. + 3;
  // lane: row (lane >> 4), slot (lane & 15) <- chunk slot ^ (row & 15)
  const int dma_r = lane >> 4;
  // fragment read for sub-step s, m-fragment i: row 16 i + r16, chunk 4 g4 + s
  const uint32_t afrag = (uint32_t)(r16 * AROW);

  for (int L = xcd * chunk + jb; L < lend; L += G8) {
    const TileRef tr = map_tile(L, p.n_tiles, p.groups, BM, p.tp, p.goff);
    const int g = tr.g;
    // rows past the group's end repeat its last row; with a gather map the rows
    // come straight from the token matrix (offsets checked to fit 32 bits)
    const uint8_t* a_base = (const uint8_t*)p.A + (p.gather ? 0 : (size_t)tr.row0 * K * 2);
    uint32_t a_off[A_INS];
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
      const int r = (w * A_INS + i) * 4 + dma_r;
      const int c = (lane & 15) ^ (r & 15);
      const int rr = min(r, tr.rows - 1);
      const uint32_t src = p.gather ? (uint32_t)p.gather[tr.row0 + rr] : (uint32_t)rr;
      a_off[i] = src * (uint32_t)K * 2u + (uint32_t)(c * 16);
    }
    // this lane's weight rows (one per n-fragment), k offset 32 g4
    const uint8_t* b_row[NF];
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      int wrow;
      const void* base;
      if (GATED) {  // fragments 0,1: gate rows; 2,3: the matching up rows
        wrow = tr.nt * 128 + w * 32 + (j & 1) * 16 + r16;
        base = (j < 2) ? p.B0 : p.B1;
      } else {
        wrow = tr.nt * 256 + w * 64 + j * 16 + r16;
        base = p.B0;
      }
      b_row[j] = (const uint8_t*)base + ((size_t)g * N * K + (size_t)wrow * K + (size_t)g4 * 32) * EB;
    }
    auto issue_a = [&](int ks) {
      uint8_t* st = As + (ks % kNST) * ASTAGE;
      const uint32_t kb = (uint32_t)min(ks, ksteps - 1) * AROW;
#pragma unroll
      for (int i = 0; i < A_INS; ++i)
        __builtin_amdgcn_global_load_lds(MOE_GPTR(a_base + a_off[i] + kb), MOE_LPTR(st + (w * A_INS + i) * 1024),
                                         16, 0, 0);
    };
    auto load_b = [&](uint4 (&dst)[NF][RAW], int ks) {
      const size_t kb = (size_t)min(ks, ksteps - 1) * kKS * EB;
#pragma unroll
      for (int j = 0; j < NF; ++j)
#pragma unroll
        for (int q = 0; q < RAW; ++q) dst[j][q] = *(const uint4*)(b_row[j] + kb + q * 16);
    };

    f32x4_t acc[MF][NF];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int j = 0; j < NF; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    constexpr int PD = FP8 ? 3 : 1;          // weight prefetch distance in steps
    constexpr int NB = NF * RAW;             // weight load instructions per wave per step
    uint4 b0[NF][RAW], b1[NF][RAW], b2[NF][RAW], b3[NF][RAW];

    // one K step: weights of `ks` in cur; weights of ks + PD requested into ahead
    // (tail steps: the compiler drops their prefetches, which no step reads, so
    // the wait there counts only the activation loads behind this step's)
    auto step = [&](int ks, uint4 (&cur)[NF][RAW], uint4 (&ahead)[NF][RAW], auto tail) {
      constexpr bool kTail = decltype(tail)::value;
      // landed: activations and weights of step ks; still in flight, newest
      // first: activations of ks + 1 and weights of ks + PD - 1 (issued one step
      // ago), and for PD = 3 the weights of ks + 1 .. ks + 2 are older than those
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(A_INS + (PD > 1 && !kTail ? NB : 0)));
      // this wave's LDS reads of step ks - 1 are complete before the barrier:
      // after it, another wave may refill that stage
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      block_sync();
      load_b(ahead, ks + PD);
      issue_fence();
      issue_a(ks + 2);
      issue_fence();
      const uint8_t* st = As + (ks % kNST) * ASTAGE;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t slot = (uint32_t)(((4 * g4 + s) ^ r16) * 16);
        bf16x8_t af[MF], bf[NF];
#pragma unroll
        for (int i = 0; i < MF; ++i) af[i] = *(const bf16x8_t*)(st + afrag + i * 16 * AROW + slot);
#pragma unroll
        for (int j = 0; j < NF; ++j) bf[j] = b_frag<FP8>(cur[j], s);
#pragma unroll
        for (int i = 0; i < MF; ++i)
#pragma unroll
          for (int j = 0; j < NF; ++j) acc[i][j] = mfma16x16x32(af[i], bf[j], acc[i][j]);
      }
    };

    block_sync();  // the previous tile's stages are free
    // Issue order matters: the waits count loads still in flight, newest first.
    // Steady state: step k issues weights(k + PD) then activations(k + 2).
    int ks = 0;
    if (PD == 3) {
      load_b(b0, 0);
      load_b(b1, 1);
      issue_fence();
      issue_a(0);
      issue_fence();
      load_b(b2, 2);
      issue_fence();
      issue_a(1);
      issue_fence();
      // ring of four: step k computes from b[k % 4] and refills b[(k + 3) % 4]
      for (; ks + 3 < ksteps; ks += 4) {
        step(ks, b0, b3, kBody);
        step(ks + 1, b1, b0, kBody);
        step(ks + 2, b2, b1, kBody);
        step(ks + 3, b3, b2, kBody);
      }
      if (ks < ksteps) step(ks, b0, b3, kTailStep);
      if (ks + 1 < ksteps) step(ks + 1, b1, b0, kTailStep);
      if (ks + 2 < ksteps) step(ks + 2, b2, b1, kTailStep);
    } else {
      issue_a(0);
      issue_fence();
      load_b(b0, 0);
      issue_fence();
      issue_a(1);
      issue_fence();
      // pairs of steps so the weight double buffer swaps roles statically
      for (; ks + 1 < ksteps; ks += 2) {
        step(ks, b0, b1, kBody);
        step(ks + 1, b1, b0, kBody);
      }
      if (ks < ksteps) step(ks, b0, b1, kTailStep);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load may land in a stage after this tile

    // ---- epilogue (rows past the group's end are not stored)
    const int rq = g4 * 4;
    if (GATED) {
      uint16_t* h = (uint16_t*)p.out;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int f = tr.nt * 128 + w * 32 + j * 16 + r16;
        float sg = 1.f, su = 1.f;
        if (FP8) { sg = ((const float*)p.S0)[(size_t)g * N + f]; su = ((const float*)p.S1)[(size_t)g * N + f]; }
#pragma unroll
        for (int i = 0; i < MF; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = i * 16 + rq + r;
            if (m < tr.rows)
              h[(size_t)(tr.row0 + m) * N + f] = f32_to_bf16_rne(silu_f32(acc[i][j][r] * sg) * (acc[i][j + 2][r] * su));
          }
      }
    } else {
      float* y = (float*)p.out;
#pragma unroll
      for (int j = 0; j < NF; ++j) {
        const int n = tr.nt * 256 + w * 64 + j * 16 + r16;
        const float sd = FP8 ? ((const float*)p.S0)[(size_t)g * N + n] : 1.f;
#pragma unroll
        for (int i = 0; i < MF; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = i * 16 + rq + r;
            if (m < tr.rows) y[(size_t)(tr.row0 + m) * N + n] = acc[i][j][r] * sd;
          }
      }
    }
  }
}

template <bool GATED, int MF>
__global__ __launch_bounds__(256, 2) void gemm_stream_int4_kernel(StreamParams p) {
  constexpr int BM = 16 * MF;
  constexpr int NF = 4;
  constexpr int AROW = kKS * 2;
  constexpr int ASTAGE = BM * AROW;
  constexpr int A_INS = BM / 16;
  constexpr int PD = 3;                    // weight prefetch distance in steps (registers allowing)
  constexpr int R = PD + 1;                // register sets in the ring
  constexpr int NBI = 2 * NF;              // loads per wave per step: codes + group words
  __shared__ __attribute__((aligned(1024))) uint8_t As[kNST * ASTAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = p.K, N = p.N, ksteps = K / kKS;
  const int total = p.n_tiles * p.tp[p.groups];
  const int G8 = gridDim.x >> 3, xcd = blockIdx.x & 7, jb = blockIdx.x >> 3;
  const int chunk = (total + 7) >> 3;
  const int lend = min(total, (xcd + 1) * chunk);
  const int g4 = lane >> 4, r16 = lane & 15;
  const int dma_r = lane >> 4;
  const uint32_t afrag = (uint32_t)(r16 * AROW);
  const size_t KB = (size_t)K / 2;         // code bytes per weight row
  const size_t KG = (size_t)K / kKS;       // group words per weight row
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

  for (int L = xcd * chunk + jb; L < lend; L += G8) {
    const TileRef tr = map_tile(L, p.n_tiles, p.groups, BM, p.tp, p.goff);
    const int g = tr.g;
    const uint8_t* a_base = (const uint8_t*)p.A + (p.gather ? 0 : (size_t)tr.row0 * K * 2);
    uint32_t a_off[A_INS];
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
      const int r = (w * A_INS + i) * 4 + dma_r;
      const int c = (lane & 15) ^ (r & 15);
      const int rr = min(r, tr.rows - 1);
      const uint32_t src = p.gather ? (uint32_t)p.gather[tr.row0 + rr] : (uint32_t)rr;
      a_off[i] = src * (uint32_t)K * 2u + (uint32_t)(c * 16);
    }
    const uint8_t* b_row[NF];
    const uint32_t* q_row[NF];
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      int wrow;
      const void* base;
      const void* qbase;
      if (GATED) {
        wrow = tr.nt * 128 + w * 32 + (j & 1) * 16 + r16;
        base = (j < 2) ? p.B0 : p.B1;
        qbase = (j < 2) ? p.S0 : p.S1;
      } else {
        wrow = tr.nt * 256 + w * 64 + j * 16 + r16;
        base = p.B0;
        qbase = p.S0;
      }
      const size_t row = (size_t)g * N + wrow;
      b_row[j] = (const uint8_t*)base + row * KB + (size_t)g4 * 16;
      q_row[j] = (const uint32_t*)qbase + row * KG;
    }
    auto issue_a = [&](int ks) {
      uint8_t* st = As + (ks % kNST) * ASTAGE;
      const uint32_t kb = (uint32_t)min(ks, ksteps - 1) * AROW;
#pragma unroll
      for (int i = 0; i < A_INS; ++i)
        __builtin_amdgcn_global_load_lds(MOE_GPTR(a_base + a_off[i] + kb), MOE_LPTR(st + (w * A_INS + i) * 1024),
                                         16, 0, 0);
    };
    auto load_w = [&](uint4 (&dw)[NF], uint32_t (&dq)[NF], int ks) {
      const int kc = min(ks, ksteps - 1);
#pragma unroll
      for (int j = 0; j < NF; ++j) dw[j] = *(const uint4*)(b_row[j] + (size_t)kc * (kKS / 2));
#pragma unroll
      for (int j = 0; j < NF; ++j) dq[j] = q_row[j][kc];
    };

    f32x4_t acc[MF][NF];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int j = 0; j < NF; ++j) acc[i][j] = zero4;
    uint4 wr[R][NF];
    uint32_t qr[R][NF];

    // one K step (= one group): codes and words of `ks` in cw / cq; those of
    // ks + PD requested into nw / nq
    auto step = [&](int ks, const uint4 (&cw)[NF], const uint32_t (&cq)[NF], uint4 (&nw)[NF], uint32_t (&nq)[NF],
                    auto tail) {
      constexpr bool kTail = decltype(tail)::value;
      // landed: everything but the newest loads -- the weights of ks + PD - 1 and
      // the activations of ks + 1, both issued one step ago
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(A_INS + (kTail ? 0 : NBI)));
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      block_sync();
      load_w(nw, nq, ks + PD);
      issue_fence();
      issue_a(ks + 2);
      issue_fence();
      const uint8_t* st = As + (ks % kNST) * ASTAGE;
      f32x4_t t[MF][NF], rs[MF];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t slot = (uint32_t)(((4 * g4 + s) ^ r16) * 16);
        bf16x8_t af[MF], bf[NF];
#pragma unroll
        for (int i = 0; i < MF; ++i) af[i] = *(const bf16x8_t*)(st + afrag + i * 16 * AROW + slot);
#pragma unroll
        for (int j = 0; j < NF; ++j) {
          const uint4 c = cw[j];
          bf[j] = int4_frag(s == 0 ? c.x : s == 1 ? c.y : s == 2 ? c.z : c.w);
        }
#pragma unroll
        for (int i = 0; i < MF; ++i) {
          rs[i] = mfma16x16x32(af[i], ones, s == 0 ? zero4 : rs[i]);
#pragma unroll
          for (int j = 0; j < NF; ++j) t[i][j] = mfma16x16x32(af[i], bf[j], s == 0 ? zero4 : t[i][j]);
        }
      }
#pragma unroll
      for (int j = 0; j < NF; ++j) {
        const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)(cq[j] & 0xFFFFu));
        const float c = (float)(128u + ((cq[j] >> 16) & 15u));
#pragma unroll
        for (int i = 0; i < MF; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(sc, fmaf(-c, rs[i][r], t[i][j][r]), acc[i][j][r]);
      }
    };

    block_sync();  // the previous tile's stages are free
    // issue order: weights 0 .. PD-2, activations 0, weights PD-1, activations 1;
    // then step k issues weights k + PD and activations k + 2
#pragma unroll
    for (int u = 0; u < PD - 1; ++u) load_w(wr[u], qr[u], u);
    issue_fence();
    issue_a(0);
    issue_fence();
    load_w(wr[PD - 1], qr[PD - 1], PD - 1);
    issue_fence();
    issue_a(1);
    issue_fence();
    // step k computes from set k % R and refills set (k + PD) % R, the one step
    // k - 1 used; whole rounds of R steps, then the remaining steps
    int ks = 0;
    for (; ks + R <= ksteps; ks += R) {
#pragma unroll
      for (int u = 0; u < R; ++u) step(ks + u, wr[u], qr[u], wr[(u + PD) % R], qr[(u + PD) % R], kBody);
    }
#pragma unroll
    for (int u = 0; u < R - 1; ++u)
      if (ks + u < ksteps) step(ks + u, wr[u], qr[u], wr[(u + PD) % R], qr[(u + PD) % R], kTailStep);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load may land in a stage after this tile

    // ---- epilogue (rows past the group's end are not stored)
    const int rq = g4 * 4;
    if (GATED) {
      uint16_t* h = (uint16_t*)p.out;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int f = tr.nt * 128 + w * 32 + j * 16 + r16;
#pragma unroll
        for (int i = 0; i < MF; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = i * 16 + rq + r;
            if (m < tr.rows) h[(size_t)(tr.row0 + m) * N + f] = f32_to_bf16_rne(silu_f32(acc[i][j][r]) * acc[i][j + 2][r]);
          }
      }
    } else {
      float* y = (float*)p.out;
#pragma unroll
      for (int j = 0; j < NF; ++j) {
        const int n = tr.nt * 256 + w * 64 + j * 16 + r16;
#pragma unroll
        for (int i = 0; i < MF; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = i * 16 + rq + r;
            if (m < tr.rows) y[(size_t)(tr.row0 + m) * N + n] = acc[i][j][r];
          }
      }
    }
  }
}

template <bool GATED, bool FP8>
moe_status launch_t(const StreamParams& p, int mf, int64_t grid, hipStream_t s) {
  if (mf == 2) hipLaunchKernelGGL((gemm_stream_kernel<GATED, FP8, 2>), dim3(grid), dim3(256), 0, s, p);
  else hipLaunchKernelGGL((gemm_stream_kernel<GATED, FP8, 4>), dim3(grid), dim3(256), 0, s, p);
  return MOE_OK;
}

}  // namespace

moe_status launch_gemm_stream(const GemmLaunch& a, const int32_t* goff, const int32_t* tp, int bm, hipStream_t s) {
  StreamParams p{a.A, a.B0, a.B1, a.S0, a.S1, a.out, goff, tp, a.groups, a.K, a.N, 0, a.gather};
  p.n_tiles = a.gated ? a.N / 128 : a.N / 256;
  const int64_t upper = (ceil_div(a.max_rows, bm) + a.groups) * p.n_tiles;
  int64_t grid = std::min<int64_t>(upper, (int64_t)device_cu_count() * 2);
  grid = ceil_div(grid, 8) * 8;
  if (grid <= 0) return MOE_OK;
  const bool fp8 = a.w_dtype == MOE_FP8_E4M3FN;
  const int mf = bm / 16;
  if (a.w_dtype == MOE_INT4) {
    const char* name = a.shared ? (a.gated ? "shared_gate_up_int4" : "shared_down_int4")
                                : (a.gated ? "gemm_gate_up_int4" : "gemm_down_int4");
    int tok = begin_launch(name, s);
    if (mf != 2) return fail(MOE_ERR_UNSUPPORTED, "INT4 weights take 32-row tiles");
    if (a.gated) hipLaunchKernelGGL((gemm_stream_int4_kernel<true, 2>), dim3(grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((gemm_stream_int4_kernel<false, 2>), dim3(grid), dim3(256), 0, s, p);
    return end_launch(tok, s);
  }
  const char* name = a.shared ? (a.gated ? (fp8 ? "shared_gate_up_fp8" : "shared_gate_up_bf16")
                                         : (fp8 ? "shared_down_fp8" : "shared_down_bf16"))
                              : (a.gated ? (fp8 ? "gemm_gate_up_fp8" : "gemm_gate_up_bf16")
                                         : (fp8 ? "gemm_down_fp8" : "gemm_down_bf16"));
  int tok = begin_launch(name, s);
  if (a.gated) {
    if (fp8) launch_t<true, true>(p, mf, grid, s);
    else launch_t<true, false>(p, mf, grid, s);
  } else {
    if (fp8) launch_t<false, true>(p, mf, grid, s);
    else launch_t<false, false>(p, mf, grid, s);
  }
  return end_launch(tok, s);
}

}  // namespace moe
