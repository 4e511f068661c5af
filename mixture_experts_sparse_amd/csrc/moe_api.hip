// C-ABI entry points of the MoE layer: host-side validation, workspace
// carving and launch sequencing.  See include/moe.h for the contract.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

namespace moe {

// ---------------------------------------------------------------- errors
namespace {
thread_local char g_err[512] = "";
}

moe_status fail(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

// ---------------------------------------------------------------- device info
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// ---------------------------------------------------------------- profiling hook
namespace {
struct ProfRec {
  const char* name;
  hipEvent_t start, stop;
};
thread_local bool g_prof = false;
thread_local std::vector<ProfRec> g_recs;
thread_local std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

int begin_launch(const char* name, hipStream_t s) {
  if (!g_prof) return -1;
  ProfRec r{name, take_event(), take_event()};
  if (!r.start || !r.stop) return -1;
  hipEventRecord(r.start, s);
  g_recs.push_back(r);
  return (int)g_recs.size() - 1;
}

moe_status end_launch(int tok, hipStream_t s) {
  const hipError_t e = hipGetLastError();
  if (tok >= 0 && tok < (int)g_recs.size()) hipEventRecord(g_recs[tok].stop, s);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

// ---------------------------------------------------------------- validation and layout
namespace {

int dtype_bytes(int dt) { return dt == MOE_F32 ? 4 : dt == MOE_BF16 ? 2 : 1; }

moe_status check_config(const moe_config* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARGUMENT, "cfg is NULL");
  if (c->T < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "T = %d < 0", c->T);
  if (c->E < 1 || c->E > 256) return fail(MOE_ERR_INVALID_ARGUMENT, "E = %d outside [1, 256]", c->E);
  if (c->top_k < 1 || c->top_k > c->E)
    return fail(MOE_ERR_INVALID_ARGUMENT, "top_k = %d outside [1, E = %d]", c->top_k, c->E);
  if (c->d <= 0 || c->F <= 0) return fail(MOE_ERR_INVALID_ARGUMENT, "d = %d, F = %d must be > 0", c->d, c->F);
  if (c->n_shared != 0 && c->n_shared != 1)
    return fail(MOE_ERR_INVALID_ARGUMENT, "n_shared = %d must be 0 or 1", c->n_shared);
  if ((int64_t)c->T * c->top_k >= (int64_t)1 << 31)
    return fail(MOE_ERR_INVALID_ARGUMENT, "T * top_k must be < 2^31");
  if (c->score != MOE_SCORE_SOFTMAX && c->score != MOE_SCORE_SIGMOID)
    return fail(MOE_ERR_INVALID_ARGUMENT, "score = %d", c->score);
  if (c->renormalize != 0 && c->renormalize != 1)
    return fail(MOE_ERR_INVALID_ARGUMENT, "renormalize = %d must be 0 or 1", c->renormalize);
  if (!(c->tau > 0.f) || !std::isfinite(c->tau))
    return fail(MOE_ERR_INVALID_ARGUMENT, "tau = %g must be finite and > 0", (double)c->tau);
  if (c->bias_mode < MOE_BIAS_NONE || c->bias_mode > MOE_BIAS_SELECT_ONLY)
    return fail(MOE_ERR_INVALID_ARGUMENT, "bias_mode = %d", c->bias_mode);
  if (c->score == MOE_SCORE_SIGMOID && (c->tau != 1.f || c->bias_mode == MOE_BIAS_LOGIT))
    return fail(MOE_ERR_UNSUPPORTED, "sigmoid scoring takes tau = 1 and no logit bias");
  if (!std::isfinite(c->capacity_factor))
    return fail(MOE_ERR_INVALID_ARGUMENT, "capacity_factor must be finite");
  if (c->act_dtype != MOE_F32 && c->act_dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARGUMENT, "act_dtype = %d", c->act_dtype);
  if (c->out_dtype != MOE_F32 && c->out_dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARGUMENT, "out_dtype = %d", c->out_dtype);
  if (c->w_dtype == MOE_F32) {
    if (c->act_dtype != MOE_F32) return fail(MOE_ERR_UNSUPPORTED, "fp32 weights need fp32 activations");
    if (c->F % 32) return fail(MOE_ERR_UNSUPPORTED, "F = %d must be a multiple of 32 for fp32 weights", c->F);
  } else if (c->w_dtype == MOE_BF16 || c->w_dtype == MOE_FP8_E4M3FN) {
    if (c->act_dtype != MOE_BF16)
      return fail(MOE_ERR_UNSUPPORTED, "bf16/fp8 weights need bf16 activations");
    if (c->F % 64) return fail(MOE_ERR_UNSUPPORTED, "F = %d must be a multiple of 64", c->F);
  } else if (c->w_dtype == MOE_INT4) {
    if (c->act_dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "INT4 weights need bf16 activations");
    if (c->F % 128 || c->d % 256)
      return fail(MOE_ERR_UNSUPPORTED, "INT4 weights need F %% 128 == 0 and d %% 256 == 0 (F = %d, d = %d)", c->F, c->d);
  } else {
    return fail(MOE_ERR_INVALID_ARGUMENT, "w_dtype = %d", c->w_dtype);
  }
  if (c->d % 128) return fail(MOE_ERR_UNSUPPORTED, "d = %d must be a multiple of 128", c->d);
  if (c->reroute_depth < 0 || c->reroute_depth > std::min(8, c->E - c->top_k))
    return fail(MOE_ERR_INVALID_ARGUMENT, "reroute_depth = %d outside [0, min(8, E - top_k)]", c->reroute_depth);
  if (c->reroute_depth > 0 && c->top_k > 64)
    return fail(MOE_ERR_UNSUPPORTED, "overflow re-routing needs top_k <= 64");
  if (c->n_groups < 0 || c->n_groups > c->E || (c->n_groups > 1 && c->E % c->n_groups))
    return fail(MOE_ERR_INVALID_ARGUMENT, "n_groups = %d must divide E = %d", c->n_groups, c->E);
  if (c->n_groups > 1) {
    if (c->topk_groups < 1 || c->topk_groups > c->n_groups)
      return fail(MOE_ERR_INVALID_ARGUMENT, "topk_groups = %d outside [1, n_groups]", c->topk_groups);
    if (c->top_k + c->reroute_depth > c->topk_groups * (c->E / c->n_groups))
      return fail(MOE_ERR_INVALID_ARGUMENT, "top_k + reroute_depth exceeds the experts of the kept groups");
  }
  return MOE_OK;
}

// C = max(1, floor(T*k/E*cf)) in double from the float32 factor; -1 = no limit.
// No expert can receive more than T*k pairs, so any C at or above that limits
// nothing: C is clamped there before the conversion, which keeps C and C*E in
// range for every finite factor without changing a result.
static_assert(sizeof(moe_config) == 17 * 4, "moe_config layout is part of the ABI");
static_assert(sizeof(moe_expert_weights) == 12 * 8, "moe_expert_weights layout is part of the ABI");

int64_t capacity_of(const moe_config* c) {
  if (!(c->capacity_factor > 0.f)) return -1;
  const double v = std::floor((double)c->T * (double)c->top_k / (double)c->E * (double)c->capacity_factor);
  const double most = std::max(1.0, (double)c->T * (double)c->top_k);
  return v < 1.0 ? 1 : (int64_t)std::min(v, most);
}

int64_t perm_rows(const moe_config* c) {
  const int64_t pairs = (int64_t)c->T * c->top_k;
  const int64_t cap = capacity_of(c);
  if (cap < 0) return pairs;
  return std::min<int64_t>(pairs, cap * c->E);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// whether a pass of this layer (routed or shared, gate/up or down) runs on the
// large-tile kernel, whose stream-K tail needs partial slots in the workspace
bool uses_stream_k(const moe_config* c) {
  for (int shared = 0; shared <= c->n_shared; ++shared)
    for (int gated = 0; gated <= 1; ++gated) {
      GemmLaunch g{};
      g.w_dtype = c->w_dtype; g.gated = gated != 0;
      g.K = gated ? c->d : c->F; g.N = gated ? c->F : c->d;
      g.groups = shared ? 1 : c->E; g.max_rows = shared ? c->T : perm_rows(c);
      if (grouped_gemm_bm(g) == 256) return true;
    }
  return false;
}

struct Layout {
  // router scratch (bf16 path): split weights, logit partials; overlaps the
  // permute / ffn scratch, which is only used after the router has finished
  int route_ep, route_split;
  size_t route_wt, route_part, route_end;
  // permute / ffn scratch
  size_t hist, reroute, tiles, tiles_sh, sk_cnt, sk_part, h, h_sh;
  // forward intermediates
  size_t logits, idx, w, counts, offsets, dest, src, ndrop, x_perm, y_perm, y_sh;
  size_t perm_end, ffn_end, total;
};

Layout layout_of(const moe_config* c) {
  Layout L{};
  const int64_t R = perm_rows(c);
  const int64_t P = (int64_t)c->T * c->top_k;
  const int64_t nblk = std::max<int64_t>(1, ceil_div(P, kPermChunk));
  const size_t hb = c->w_dtype == MOE_F32 ? 4 : 2;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  route_plan(c->T, c->d, c->E, c->act_dtype, &L.route_ep, &L.route_split);
  L.route_wt = take(sizeof(uint16_t) * 3 * (size_t)L.route_ep * c->d);
  L.route_part = take(sizeof(float) * (size_t)L.route_split * c->T * L.route_ep);
  L.route_end = o;
  o = 0;
  // scratch shared by moe_permute and moe_expert_ffn (they never run concurrently
  // on one workspace within moe_forward; standalone callers pass one each)
  L.hist = take(sizeof(int32_t) * nblk * c->E);
  L.reroute = take(c->reroute_depth > 0 ? sizeof(int32_t) * reroute_ws_ints(c->T, c->top_k, c->E, c->reroute_depth) : 0);
  L.perm_end = o;
  L.tiles = take(sizeof(int32_t) * tile_list_ints(c->E, R));
  L.tiles_sh = take(sizeof(int32_t) * tile_list_ints(1, c->T));
  // stream-K tail of the large-tile down passes: counters and partial slots
  // (reused by the shared expert's passes, which run after the routed ones)
  L.sk_cnt = take(sizeof(int32_t) * kSkUnits);
  L.sk_part = take(uses_stream_k(c) ? sizeof(float) * (size_t)std::min(device_cu_count(), kSkUnits) * 65536 : 0);
  L.h = take(hb * R * c->F);
  L.h_sh = take(c->n_shared ? hb * (size_t)c->T * c->F : 0);
  L.ffn_end = o;
  o = std::max(L.ffn_end, L.route_end);
  L.logits = take(sizeof(float) * (size_t)c->T * c->E);
  L.idx = take(sizeof(int32_t) * (size_t)c->T * (c->top_k + c->reroute_depth));
  L.w = take(sizeof(float) * P);
  L.counts = take(sizeof(int32_t) * c->E);
  L.offsets = take(sizeof(int32_t) * (c->E + 1));
  L.dest = take(sizeof(int32_t) * P);
  L.src = take(sizeof(int32_t) * std::max<int64_t>(R, 1));
  L.ndrop = take(sizeof(int32_t));
  L.x_perm = take((size_t)dtype_bytes(c->act_dtype) * R * c->d);
  L.y_perm = take(sizeof(float) * R * c->d);
  L.y_sh = take(c->n_shared ? sizeof(float) * (size_t)c->T * c->d : 0);
  // moe_router_stats reuses the workspace for its per-block partial sums
  L.total = std::max(o, (size_t)router_stats_ws_bytes(c->T, c->E));
  return L;
}

moe_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return MOE_OK;
  if (!ws) return fail(MOE_ERR_INVALID_ARGUMENT, "workspace is NULL (%zu bytes needed)", need);
  if ((uintptr_t)ws & 255u) return fail(MOE_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (have < need) return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", have, need);
  return MOE_OK;
}

moe_status check_weights(const moe_config* c, const moe_expert_weights* w) {
  if (!w) return fail(MOE_ERR_INVALID_ARGUMENT, "weights is NULL");
  if (!w->w_gate || !w->w_up || !w->w_down) return fail(MOE_ERR_INVALID_ARGUMENT, "expert weight pointer is NULL");
  if (!aligned16(w->w_gate) || !aligned16(w->w_up) || !aligned16(w->w_down))
    return fail(MOE_ERR_INVALID_ARGUMENT, "expert weights must be 16-byte aligned");
  const bool scaled = c->w_dtype == MOE_FP8_E4M3FN || c->w_dtype == MOE_INT4;
  if (scaled != (w->s_gate && w->s_up && w->s_down) || (!scaled && (w->s_gate || w->s_up || w->s_down)))
    return fail(MOE_ERR_INVALID_ARGUMENT, "scales are required for fp8 and INT4 weights and only for them");
  if (c->w_dtype == MOE_INT4 && (!aligned4(w->s_gate) || !aligned4(w->s_up) || !aligned4(w->s_down)))
    return fail(MOE_ERR_INVALID_ARGUMENT, "INT4 group words must be 4-byte aligned");
  if (c->n_shared) {
    if (!w->sh_gate || !w->sh_up || !w->sh_down) return fail(MOE_ERR_INVALID_ARGUMENT, "shared expert weights missing");
    if (!aligned16(w->sh_gate) || !aligned16(w->sh_up) || !aligned16(w->sh_down))
      return fail(MOE_ERR_INVALID_ARGUMENT, "shared expert weights must be 16-byte aligned");
    if (scaled != (w->sh_s_gate && w->sh_s_up && w->sh_s_down) ||
        (!scaled && (w->sh_s_gate || w->sh_s_up || w->sh_s_down)))
      return fail(MOE_ERR_INVALID_ARGUMENT, "shared expert scales are required for fp8 and INT4 weights and only for them");
    if (c->w_dtype == MOE_INT4 && (!aligned4(w->sh_s_gate) || !aligned4(w->sh_s_up) || !aligned4(w->sh_s_down)))
      return fail(MOE_ERR_INVALID_ARGUMENT, "INT4 group words must be 4-byte aligned");
  } else if (w->sh_gate || w->sh_up || w->sh_down) {
    return fail(MOE_ERR_INVALID_ARGUMENT, "shared expert weights given but n_shared == 0");
  }
  return MOE_OK;
}

moe_status check_route_args(const moe_config* c, const void* x, const float* w_router, const float* bias,
                            const float* gumbel_u, const int32_t* topk_idx, const float* topk_w) {
  if (c->T > 0) {
    if (!x || !w_router || !topk_idx || !topk_w) return fail(MOE_ERR_INVALID_ARGUMENT, "route pointer is NULL");
    if (!aligned16(x)) return fail(MOE_ERR_INVALID_ARGUMENT, "x must be 16-byte aligned");
  }
  if ((c->bias_mode != MOE_BIAS_NONE) != (bias != nullptr))
    return fail(MOE_ERR_INVALID_ARGUMENT, "bias must be given exactly when bias_mode != NONE");
  if (gumbel_u && c->score != MOE_SCORE_SOFTMAX)
    return fail(MOE_ERR_UNSUPPORTED, "Gumbel noise applies to softmax scoring only");
  return MOE_OK;
}

// ---- step runners shared by the standalone entry points and moe_forward
moe_status run_route(const moe_config* c, const void* x, const float* w_router, const float* bias,
                     const float* gumbel_u, float* logits, int32_t* topk_idx, float* topk_w, char* ws,
                     hipStream_t s) {
  RouteLaunch r{x, w_router, bias, gumbel_u, logits, topk_idx, topk_w, c->T, c->d, c->E, c->top_k,
                c->score, c->renormalize, c->bias_mode, c->act_dtype, c->tau};
  const Layout L = layout_of(c);
  r.fb = c->reroute_depth;
  r.n_groups = c->n_groups > 1 ? c->n_groups : 0;
  r.topk_groups = c->topk_groups;
  r.ep = L.route_ep;
  r.split = L.route_split;
  r.wt = (uint16_t*)(ws + L.route_wt);
  r.part = (float*)(ws + L.route_part);
  return launch_route(r, s);
}

// tiles / tile_bm: also write the routed gate/up GEMM's tile lists (moe_forward),
// which the permute does unless overflow re-routing moves rows after its scan
moe_status run_permute(const moe_config* c, const void* x, const int32_t* topk_idx, int32_t* counts,
                       int32_t* offsets, int32_t* dest_row, int32_t* src_token, int32_t* n_dropped,
                       void* x_perm, int32_t* stats, char* ws, hipStream_t s, int32_t* tiles = nullptr,
                       int tile_bm = 0) {
  const Layout L = layout_of(c);
  PermuteLaunch p{x, topk_idx, counts, offsets, dest_row, src_token, n_dropped, x_perm, stats,
                  (int32_t*)(ws + L.hist), c->T, c->d, c->E, c->top_k, dtype_bytes(c->act_dtype),
                  capacity_of(c), perm_rows(c)};
  p.fb = c->reroute_depth;
  p.reroute = (int32_t*)(ws + L.reroute);
  p.tiles = tiles;
  p.tile_bm = tile_bm;
  p.sk_zero = tiles ? (int32_t*)(ws + L.sk_cnt) : nullptr;
  return launch_permute(p, s);
}

// The routed gate/up pass: A = x_perm, or A = x read through `gather` (src_token).
GemmLaunch gate_up_launch(const moe_config* c, const void* x, const void* x_perm, const int32_t* gather,
                          const int32_t* offsets, const moe_expert_weights* w, char* ws) {
  const Layout L = layout_of(c);
  GemmLaunch g{};
  g.w_dtype = c->w_dtype;
  g.A = gather ? x : x_perm; g.gather = gather;
  g.B0 = w->w_gate; g.B1 = w->w_up; g.S0 = w->s_gate; g.S1 = w->s_up;
  g.out = ws + L.h; g.offsets = offsets; g.tile_prefix = (int32_t*)(ws + L.tiles);
  g.groups = c->E; g.single_rows = 0; g.max_rows = perm_rows(c); g.K = c->d; g.N = c->F; g.gated = true;
  // with re-routing a group still holds at most C rows
  g.group_rows_max = capacity_of(c) >= 0 ? std::min<int64_t>(capacity_of(c), g.max_rows) : g.max_rows;
  g.sk_cnt = (int32_t*)(ws + L.sk_cnt);
  g.sk_part = uses_stream_k(c) ? (float*)(ws + L.sk_part) : nullptr;
  return g;
}

// gather: src_token when the gate/up pass reads x directly (x_perm is then unused).
// tiles_ready: the permute already wrote the gate/up pass's tile lists
moe_status run_ffn(const moe_config* c, const void* x, const void* x_perm, const int32_t* gather,
                   const int32_t* offsets, const moe_expert_weights* w, float* y_perm, float* y_shared, char* ws,
                   hipStream_t s, bool tiles_ready = false) {
  if (c->T == 0) return MOE_OK;
  const Layout L = layout_of(c);
  // routed experts: gate/up pass then down pass
  GemmLaunch g = gate_up_launch(c, x, x_perm, gather, offsets, w, ws);
  g.tiles_ready = tiles_ready;
  moe_status st = launch_grouped_gemm(g, s);
  if (st != MOE_OK) return st;
  const int bm_gate_up = grouped_gemm_bm(g);
  g.A = ws + L.h; g.gather = nullptr; g.B0 = w->w_down; g.B1 = nullptr; g.S0 = w->s_down; g.S1 = nullptr;
  g.out = y_perm; g.K = c->F; g.N = c->d; g.gated = false;
  g.tiles_ready = grouped_gemm_bm(g) == bm_gate_up;  // same offsets and rows: reuse the tile lists
  st = launch_grouped_gemm(g, s);
  if (st != MOE_OK || !c->n_shared) return st;
  // shared expert over all tokens
  g.A = x; g.B0 = w->sh_gate; g.B1 = w->sh_up; g.S0 = w->sh_s_gate; g.S1 = w->sh_s_up;
  g.out = ws + L.h_sh; g.offsets = nullptr; g.tile_prefix = (int32_t*)(ws + L.tiles_sh);
  g.groups = 1; g.single_rows = c->T; g.max_rows = c->T; g.K = c->d; g.N = c->F; g.gated = true;
  g.shared = true; g.tiles_ready = false; g.group_rows_max = c->T;
  st = launch_grouped_gemm(g, s);
  if (st != MOE_OK) return st;
  const int bm_sh = grouped_gemm_bm(g);
  g.A = ws + L.h_sh; g.B0 = w->sh_down; g.B1 = nullptr; g.S0 = w->sh_s_down; g.S1 = nullptr;
  g.out = y_shared; g.K = c->F; g.N = c->d; g.gated = false;
  g.tiles_ready = grouped_gemm_bm(g) == bm_sh;
  return launch_grouped_gemm(g, s);
}

moe_status run_combine(const moe_config* c, const float* y_perm, const float* y_shared,
                       const int32_t* dest_row, const float* topk_w, void* out, hipStream_t s) {
  const CombineLaunch cl{y_perm, c->n_shared ? y_shared : nullptr, dest_row, topk_w, out, c->T, c->d, c->top_k,
                         c->out_dtype};
  return launch_combine(cl, s, perm_rows(c));
}

// ---- the allocation-free forward's scratch: one array per device, in the
// library's code object, whose device address is looked up once per device
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // per device ordinal: the array's address, or null until looked up

moe_status scratch_address(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_UNSUPPORTED, "device ordinal %d: at most 64 devices", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (r != hipSuccess || !p)
      return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(r));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_err; }

int32_t moe_version(void) { return 200; }

moe_status moe_workspace_bytes(const moe_config* cfg, size_t* bytes) {
  g_err[0] = 0;
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = layout_of(cfg).total;
  return MOE_OK;
}

moe_status moe_permuted_rows(const moe_config* cfg, int64_t* rows) {
  g_err[0] = 0;
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!rows) return fail(MOE_ERR_INVALID_ARGUMENT, "rows is NULL");
  *rows = perm_rows(cfg);
  return MOE_OK;
}

moe_status moe_route(const moe_config* cfg, const void* x, const float* w_router, const float* bias,
                     const float* gumbel_u, float* logits, int32_t* topk_idx, float* topk_w, void* ws,
                     size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  moe_status st = check_config(cfg);
  if (st == MOE_OK) st = check_route_args(cfg, x, w_router, bias, gumbel_u, topk_idx, topk_w);
  if (st != MOE_OK) return st;
  if (cfg->T > 0) {
    st = check_ws(ws, ws_bytes, layout_of(cfg).route_end);
    if (st != MOE_OK) return st;
  }
  return run_route(cfg, x, w_router, bias, gumbel_u, logits, topk_idx, topk_w, (char*)ws, (hipStream_t)stream);
}

moe_status moe_permute(const moe_config* cfg, const void* x, const int32_t* topk_idx, int32_t* counts,
                       int32_t* offsets, int32_t* dest_row, int32_t* src_token, int32_t* n_dropped,
                       void* x_perm, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!counts || !offsets || !n_dropped) return fail(MOE_ERR_INVALID_ARGUMENT, "permute output pointer is NULL");
  if (cfg->T > 0) {
    if (!x || !topk_idx || !dest_row || !src_token || !x_perm)
      return fail(MOE_ERR_INVALID_ARGUMENT, "permute pointer is NULL");
    if (!aligned16(x) || !aligned16(x_perm)) return fail(MOE_ERR_INVALID_ARGUMENT, "x and x_perm must be 16-byte aligned");
  }
  st = check_ws(ws, ws_bytes, layout_of(cfg).perm_end);
  if (st != MOE_OK) return st;
  return run_permute(cfg, x, topk_idx, counts, offsets, dest_row, src_token, n_dropped, x_perm, nullptr,
                     (char*)ws, (hipStream_t)stream);
}

moe_status moe_expert_ffn(const moe_config* cfg, const void* x, const void* x_perm, const int32_t* offsets,
                          const moe_expert_weights* weights, float* y_perm, float* y_shared, void* ws,
                          size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  moe_status st = check_config(cfg);
  if (st == MOE_OK) st = check_weights(cfg, weights);
  if (st != MOE_OK) return st;
  if (cfg->T > 0) {
    if (!x_perm || !offsets || !y_perm) return fail(MOE_ERR_INVALID_ARGUMENT, "expert_ffn pointer is NULL");
    if (!aligned16(x_perm) || !aligned16(y_perm)) return fail(MOE_ERR_INVALID_ARGUMENT, "x_perm and y_perm must be 16-byte aligned");
    if (cfg->n_shared && (!x || !y_shared || !aligned16(x) || !aligned16(y_shared)))
      return fail(MOE_ERR_INVALID_ARGUMENT, "x and y_shared (16-byte aligned) are required with a shared expert");
  }
  st = check_ws(ws, ws_bytes, layout_of(cfg).ffn_end);
  if (st != MOE_OK) return st;
  return run_ffn(cfg, x, x_perm, nullptr, offsets, weights, y_perm, y_shared, (char*)ws,
                 (hipStream_t)stream);
}

moe_status moe_combine(const moe_config* cfg, const float* y_perm, const float* y_shared, const int32_t* dest_row,
                       const float* topk_w, void* out, void* stream) {
  g_err[0] = 0;
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->T > 0) {
    if (!y_perm || !dest_row || !topk_w || !out) return fail(MOE_ERR_INVALID_ARGUMENT, "combine pointer is NULL");
    if (!aligned16(y_perm) || !aligned16(out)) return fail(MOE_ERR_INVALID_ARGUMENT, "y_perm and out must be 16-byte aligned");
    if (cfg->n_shared && (!y_shared || !aligned16(y_shared)))
      return fail(MOE_ERR_INVALID_ARGUMENT, "y_shared (16-byte aligned) is required with a shared expert");
  }
  return run_combine(cfg, y_perm, y_shared, dest_row, topk_w, out, (hipStream_t)stream);
}

moe_status moe_forward(const moe_config* cfg, const void* x, const float* w_router, const float* bias,
                       const float* gumbel_u, const moe_expert_weights* weights, void* out, int32_t* stats,
                       const moe_routing_out* routing, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  moe_status st = check_config(cfg);
  if (st == MOE_OK) st = check_weights(cfg, weights);
  if (st != MOE_OK) return st;
  // placeholders for the route check: real pointers come from the workspace
  static const int32_t dummy_i = 0;
  static const float dummy_f = 0.f;
  st = check_route_args(cfg, x, w_router, bias, gumbel_u, &dummy_i, &dummy_f);
  if (st != MOE_OK) return st;
  if (cfg->T > 0 && (!out || !aligned16(out))) return fail(MOE_ERR_INVALID_ARGUMENT, "out must be non-NULL and 16-byte aligned");
  const Layout L = layout_of(cfg);
  st = check_ws(ws, ws_bytes, L.total);
  if (st != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  float* logits = (routing && routing->logits) ? routing->logits : (float*)(w + L.logits);
  int32_t* idx = (routing && routing->topk_idx) ? routing->topk_idx : (int32_t*)(w + L.idx);
  float* tw = (routing && routing->topk_w) ? routing->topk_w : (float*)(w + L.w);
  int32_t* dest = (routing && routing->dest_row) ? routing->dest_row : (int32_t*)(w + L.dest);
  int32_t* counts = (int32_t*)(w + L.counts);
  int32_t* offsets = (int32_t*)(w + L.offsets);
  int32_t* src = (int32_t*)(w + L.src);
  int32_t* ndrop = (int32_t*)(w + L.ndrop);
  void* x_perm = w + L.x_perm;
  float* y_perm = (float*)(w + L.y_perm);
  float* y_sh = cfg->n_shared ? (float*)(w + L.y_sh) : nullptr;

  st = run_route(cfg, x, w_router, bias, gumbel_u, (routing && routing->logits) ? logits : nullptr, idx, tw, w, s);
  if (st != MOE_OK) return st;
  // gather fusion: when the gate/up kernel can read the token rows through
  // src_token, the permute writes no x_perm and the rows are read once, by the GEMM
  const GemmLaunch gu = gate_up_launch(cfg, x, x_perm, src, offsets, weights, w);
  const bool gather = cfg->T > 0 && gather_ok(gu, cfg->T);
  // the permute's scan block also writes the gate/up tile lists, unless
  // re-routing moves rows after it
  const bool tiles_in_permute = cfg->T > 0 && !(cfg->reroute_depth > 0 && capacity_of(cfg) >= 0);
  st = run_permute(cfg, x, idx, counts, offsets, dest, src, ndrop, gather ? nullptr : x_perm, stats, w, s,
                   tiles_in_permute ? (int32_t*)(w + layout_of(cfg).tiles) : nullptr, grouped_gemm_bm(gu));
  if (st != MOE_OK) return st;
  st = run_ffn(cfg, x, x_perm, gather ? src : nullptr, offsets, weights, y_perm, y_sh, w, s, tiles_in_permute);
  if (st != MOE_OK) return st;
  return run_combine(cfg, y_perm, y_sh, dest, tw, out, s);
}

moe_status moe_forward_noalloc(const moe_config* cfg, const void* x, const float* w_router, const float* bias,
                               const float* gumbel_u, const moe_expert_weights* weights, void* out, int32_t* stats,
                               const moe_routing_out* routing, void* stream) {
  g_err[0] = 0;
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  const size_t need = layout_of(cfg).total;
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_UNSUPPORTED,
                "this layer needs %zu bytes of scratch; moe_forward_noalloc holds %zu per device "
                "(call moe_forward with a workspace instead)",
                need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != MOE_OK) return st;
  return moe_forward(cfg, x, w_router, bias, gumbel_u, weights, out, stats, routing, ws,
                     (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}

moe_status moe_router_stats(const moe_config* cfg, const float* logits, const float* bias,
                            const float* gumbel_u, const int32_t* counts, float* prob_mean, float* aux,
                            void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!counts || !prob_mean) return fail(MOE_ERR_INVALID_ARGUMENT, "counts and prob_mean must be non-NULL");
  if (cfg->T > 0 && !logits) return fail(MOE_ERR_INVALID_ARGUMENT, "logits is NULL");
  if (cfg->T > 0 && cfg->bias_mode == MOE_BIAS_LOGIT && !bias)
    return fail(MOE_ERR_INVALID_ARGUMENT, "a logit bias needs the bias vector");
  if (gumbel_u && cfg->score != MOE_SCORE_SOFTMAX)
    return fail(MOE_ERR_INVALID_ARGUMENT, "Gumbel noise needs softmax scoring");
  st = check_ws(ws, ws_bytes, (size_t)router_stats_ws_bytes(cfg->T, cfg->E));
  if (st != MOE_OK) return st;
  RouterStatsLaunch a{logits, bias, gumbel_u, counts, prob_mean, aux, (double*)ws, cfg->T, cfg->E, cfg->score,
                      cfg->bias_mode, cfg->tau};
  return launch_router_stats(a, (hipStream_t)stream);
}

moe_status moe_bias_update(const moe_config* cfg, const int32_t* counts, float* bias, float decay, float rate,
                           void* stream) {
  g_err[0] = 0;
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!counts || !bias) return fail(MOE_ERR_INVALID_ARGUMENT, "counts and bias must be non-NULL");
  if (!std::isfinite(decay) || !std::isfinite(rate))
    return fail(MOE_ERR_INVALID_ARGUMENT, "decay = %g and rate = %g must be finite", (double)decay, (double)rate);
  return launch_bias_update(counts, bias, cfg->E, decay, rate, (hipStream_t)stream);
}

moe_status moe_profile_enable(int32_t on) {
  g_prof = on != 0;
  return MOE_OK;
}

moe_status moe_profile_read(moe_kernel_time* out, int32_t max_entries, int32_t* n_entries) {
  g_err[0] = 0;
  if (!n_entries || (max_entries > 0 && !out)) return fail(MOE_ERR_INVALID_ARGUMENT, "output pointer is NULL");
  std::vector<moe_kernel_time> acc;
  for (const ProfRec& r : g_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      ms = 0.f;
    moe_kernel_time* slot = nullptr;
    for (auto& a : acc)
      if (std::strncmp(a.name, r.name, sizeof(a.name)) == 0) slot = &a;
    if (!slot) {
      moe_kernel_time t{};
      std::snprintf(t.name, sizeof(t.name), "%s", r.name);
      acc.push_back(t);
      slot = &acc.back();
    }
    slot->launches += 1;
    slot->total_ms += ms;
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_recs.clear();
  const int n = (int)acc.size();
  for (int i = 0; i < n && i < max_entries; ++i) out[i] = acc[i];
  *n_entries = n;
  return MOE_OK;
}

}  // extern "C"
