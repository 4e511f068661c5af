/*
 * moe.h -- C ABI of the sparse Mixture-of-Experts layer for AMD MI355X (gfx950).
 *
 * The layer has five steps; each entry point below runs one or all of them as
 * hand-written HIP kernels on the caller's stream:
 *
 *   moe_route      router GEMM z = x W_r, score (softmax keys with optional
 *                  logit bias, Gumbel noise and temperature, or sigmoid with a
 *                  selection-only bias), wavefront top-k, gate weights
 *   moe_permute    per-expert histogram, exclusive scan, capacity limit with
 *                  first-come-first-kept drops, stable permutation, row scatter
 *   moe_expert_ffn grouped SwiGLU FFN of every expert over its rows on bf16
 *                  MFMA (fp8 e4m3fn weights decoded exactly to bf16; fp32 path
 *                  for fp32 weights), plus the optional always-on shared expert
 *   moe_combine    out[t] = sum_j w[t,j] * y[dest_row[t,j]] (+ y_shared[t])
 *   moe_forward    all of the above, back to back, with no host synchronisation
 *
 * Sources (pages cited by title, host and section):
 *  [P1] "GPT-4 has 1.8T parameters but uses 2% per token: dynamic sparse
 *       activation" (mlqm.cn): s3.1 gating network with Gumbel noise and
 *       temperature, s3.3 SwiGLU experts, s4.2 sparse-MoE model code.
 *  [P2] "Parameter scale and the truth about sparse activation"
 *       (deepseek.csdn.net): s3.1 top-k routing and temperature, s3.2 expert
 *       capacity = tokens * k / experts * capacity_factor (at least 1),
 *       overflow marking; s5.1 deterministic-router switch for the Gumbel noise.
 *  [P3] "MoE sparse activation: principles and engineering practice"
 *       (kapook.pages.dev mirror of blog.csdn.net): s3.1 bias-free linear
 *       router, sorted top-k, softmax over the chosen logits, weighted sum of
 *       expert outputs; s3.2 experts share one shape; s4.2 expert fusion
 *       (one matmul per expert over its tokens).
 *  [P4] "V4 full-stack architecture" (kwkr.cn): s2.2 fine-grained and shared
 *       experts; the 256-expert top-8 configuration.
 *  [P5] "From sparse MoE to conditional memory" (m.nxbn.cn): dynamic routing
 *       with a per-expert bias, the gating-network code (top-k on biased
 *       scores), the fused gather / expert / weighted-sum forward signature.
 *
 * Conventions for every entry point
 *  - Tensor pointers are DEVICE pointers, row-major, owned by the caller.  The
 *    library allocates and frees nothing, keeps no pointer after returning and
 *    never synchronises the stream.  Work is enqueued on `stream` (a
 *    hipStream_t; NULL = the null stream); buffers must stay valid until the
 *    stream has consumed them.
 *  - Every argument is validated on the host before anything is launched.  A
 *    failed check returns a non-zero moe_status and launches nothing;
 *    moe_last_error() then holds a thread-local description.  No C++
 *    exception crosses this interface.
 *  - Results are deterministic: no atomic decides any order or any sum, so two
 *    calls on the same inputs give bit-identical outputs.
 *  - Entry points may be called from several host threads at once.  Calls
 *    that run concurrently (on different streams) need workspaces and output
 *    buffers of their own; calls that share a workspace must be ordered on one
 *    stream.
 *  - Expert weights are stored [out, in] (reduction dimension contiguous):
 *    W_gate, W_up are [E, F, d], W_down is [E, d, F].  fp8 weights are OCP
 *    e4m3fn codes with one float32 scale per output row ([E,F], [E,F], [E,d]).
 *  - Limits: 1 <= top_k <= E <= 256; T >= 0 (T = 0 is a no-op);
 *    d % 128 == 0 always; F % 64 == 0 for bf16/fp8 weights, F % 32 == 0
 *    for fp32 weights; T * top_k < 2^31.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,  /* null pointer, bad size, bad enum value       */
  MOE_ERR_UNSUPPORTED = 2,       /* valid but not implemented combination         */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4                /* a HIP launch or runtime call failed           */
} moe_status;

/* MOE_INT4 (expert weights only): group-wise 4-bit weights ([P3] s4.2
 * quantisation: every 128 weights along a row's input dimension form a group
 * with its own scale and zero point; w = scale * (q - zero)). */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3FN = 2, MOE_INT4 = 3 } moe_dtype;
typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score;
typedef enum {
  MOE_BIAS_NONE = 0,
  MOE_BIAS_LOGIT = 1,        /* softmax only: b is added to the logits (enters the weights) */
  MOE_BIAS_SELECT_ONLY = 2   /* b is added to the keys only; weights use unbiased scores    */
} moe_bias_mode;

/* Problem description shared by all entry points.  All fields are 32-bit. */
typedef struct {
  int32_t T;                 /* tokens                                                    */
  int32_t d;                 /* hidden size                                               */
  int32_t E;                 /* routed experts, 1..256                                    */
  int32_t top_k;             /* experts per token, 1..E                                   */
  int32_t F;                 /* expert inner size (also the shared expert's)              */
  int32_t n_shared;          /* always-on shared experts: 0 or 1 (added with weight 1)    */
  int32_t score;             /* moe_score                                                 */
  int32_t renormalize;       /* 1: gate weights renormalised over the chosen k;           */
                             /* 0: softmax over all E (sigmoid: raw scores)               */
  float tau;                 /* temperature > 0 (softmax only; sigmoid requires 1)        */
  int32_t bias_mode;         /* moe_bias_mode                                             */
  float capacity_factor;     /* <= 0: no limit; else C = max(1, floor(T*k/E*cf))          */
  int32_t act_dtype;         /* x: MOE_F32 or MOE_BF16                                    */
  int32_t w_dtype;           /* expert weights: MOE_F32 (requires act F32), MOE_BF16,     */
                             /* MOE_FP8_E4M3FN (requires act BF16), MOE_INT4 (requires    */
                             /* act BF16, F % 128 == 0 and d % 256 == 0)                  */
  int32_t out_dtype;         /* layer output: MOE_F32 or MOE_BF16                         */
  int32_t reroute_depth;     /* overflow re-routing ([P2] s3.2 level 2): 0 = off, else D  */
                             /* in 1 .. min(8, E - top_k) fallback experts per token;      */
                             /* needs top_k <= 64; acts only under a capacity limit        */
  int32_t n_groups;          /* group-limited routing ([P3] closing case: the group first, */
                             /* then the router inside it): 0 or 1 = off; else the experts */
                             /* form n_groups contiguous blocks (n_groups divides E)       */
  int32_t topk_groups;       /* groups kept per token: the ones with the largest maximum   */
                             /* key, ties to the lower group; the top-k (and fallbacks)    */
                             /* come from their experts: top_k + reroute_depth <=          */
                             /* topk_groups * E / n_groups                                 */
} moe_config;

/* Expert weights, row-major per expert: w_gate, w_up [E,F,d], w_down [E,d,F]
 * (a row holds one output's weights over the input dimension), 16-byte aligned.
 *   MOE_F32 / MOE_BF16: one element per weight; the s_* members NULL.
 *   MOE_FP8_E4M3FN: one OCP e4m3fn code byte per weight; s_* = f32 scale per
 *     row ([E,F] for gate/up, [E,d] for down), w = scale * decode(code).
 *   MOE_INT4: two codes per byte, [E,F,d/2] and [E,d,F/2], the even input index
 *     in the low nibble; s_* = one uint32 word per 128-weight group of a row
 *     ([E,F,d/128], [E,d,F/128]; 4-byte aligned): bits 0..15 the fp16 scale,
 *     bits 16..19 the zero point z, the rest ignored; w = scale * (q - z).
 * The sh_* members describe the shared expert (E = 1 in the shapes above, same
 * dtype) and must be non-NULL exactly when n_shared == 1. */
typedef struct {
  const void* w_gate;  const void* w_up;  const void* w_down;
  const void* s_gate;  const void* s_up;  const void* s_down;
  const void* sh_gate; const void* sh_up; const void* sh_down;
  const void* sh_s_gate; const void* sh_s_up; const void* sh_s_down;
} moe_expert_weights;

/* Optional routing outputs of moe_forward (any member may be NULL). */
typedef struct {
  float* logits;       /* [T,E] f32 router logits z                                  */
  int32_t* topk_idx;   /* [T,k+D] chosen experts, descending key, ties -> lower index, */
                       /* then the D = reroute_depth fallback experts               */
  float* topk_w;       /* [T,k] gate weights                                          */
  int32_t* dest_row;   /* [T,k] permuted row of each pair, -1 when dropped            */
} moe_routing_out;

/* Static description of a status code (never NULL). */
const char* moe_status_string(moe_status s);

/* Thread-local detail of the last failure on the calling thread ("" if none). */
const char* moe_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t moe_version(void);

/* Device workspace, in bytes, that moe_route / moe_permute / moe_expert_ffn /
 * moe_forward need for `cfg` on the current device (each entry point needs at
 * most this much; the split of the work across compute units, and so the size,
 * depends on the device).  The pointer passed as `ws` must be 256-byte aligned.
 * Returns a status; *bytes is set only on MOE_OK. */
moe_status moe_workspace_bytes(const moe_config* cfg, size_t* bytes);

/* Rows of the permuted buffers (x_perm, y_perm, src_token) the caller must
 * provide: T*k, or min(T*k, E*C) under a capacity limit. */
moe_status moe_permuted_rows(const moe_config* cfg, int64_t* rows);

/* Steps 1-2: router GEMM, keys, top-k and gate weights ([P3] s3.1, [P1] s3.1,
 * [P5] gating network, [P2] s3.1).
 *   x          [T,d] act_dtype
 *   w_router   [d,E] f32
 *   bias       [E] f32; required iff bias_mode != NONE
 *   gumbel_u   [T,E] f32 uniforms in (0,1), or NULL for a deterministic router
 *              ([P2] s5.1); softmax only.  Noise g = -log(-log u) is added to the
 *              (biased) logits before the temperature: l = (z + b + g) / tau.
 *   logits     [T,E] f32 output z, or NULL
 *   topk_idx   [T,k+D] int32 output (D = reroute_depth: the next-best experts
 *              after the top-k, in key order);  topk_w [T,k] f32 output
 *   ws, ws_bytes  device workspace (bf16 x: split router weights and logit
 *              partials; fp32 x needs none and may pass NULL) */
moe_status moe_route(const moe_config* cfg, const void* x, const float* w_router,
                     const float* bias, const float* gumbel_u, float* logits,
                     int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                     void* stream);

/* Steps 3-4: capacity and permutation ([P2] s3.2; [P3] s4.2; [P5] dynamic
 * routing -- the tensor reorganised by routing index).  Pairs (t,j) are ranked
 * per expert in (t,j) order; a pair is kept iff its rank < C.  Kept pairs of
 * expert e occupy rows offsets[e] .. offsets[e+1]-1 in token order.
 *   x          [T,d] act_dtype;  topk_idx [T,k+D] int32 in [0,E)
 *   counts     [E]   int32 out: pairs routed to each expert (before the limit)
 *   offsets    [E+1] int32 out: exclusive scan of kept = min(counts, C)
 *   dest_row   [T,k] int32 out: row of each pair, -1 when dropped
 *   src_token  [R]   int32 out: token of each row, -1 for rows >= offsets[E]
 *   n_dropped  [1]   int32 out
 *   x_perm     [R,d] act_dtype out: x_perm[dest_row[t,j]] = x[t]
 *   (R = moe_permuted_rows(cfg)); ws, ws_bytes: device workspace */
/* Overflow re-routing (reroute_depth = D > 0 with a capacity limit; [P2] s3.2
 * level 2: an overflowed token goes to its next-best expert that is not full):
 * topk_idx then has k + D columns, the top-k followed by the D next-best
 * experts in key order (moe_route writes them).  After the first pass, the
 * dropped pairs are visited in (t,j) order and each takes the first of its
 * token's D fallback experts that holds fewer than C pairs and does not already
 * serve the token; none -> it stays dropped.  A re-routed pair keeps its gate
 * weight.  Expert e's rows: its first-pass pairs in (t,j) order, then its
 * re-routed pairs in (t,j) order.  counts stay the requested counts; offsets
 * (and moe_forward's kept) count the final rows; n_dropped the pairs left
 * without an expert. */
moe_status moe_permute(const moe_config* cfg, const void* x, const int32_t* topk_idx,
                       int32_t* counts, int32_t* offsets, int32_t* dest_row,
                       int32_t* src_token, int32_t* n_dropped, void* x_perm,
                       void* ws, size_t ws_bytes, void* stream);

/* Step 5: the experts ([P1] s3.3 SwiGLU; [P3] s4.2 expert fusion; [P4] s2.2
 * shared expert).  For each expert e and each row r in [offsets[e], offsets[e+1]):
 *   y_perm[r] = (silu(x_perm[r] W_gate[e]^T) * (x_perm[r] W_up[e]^T)) W_down[e]^T
 * with f32 accumulation; the inner activation h is rounded to bf16 (f32 for
 * fp32 weights).  y_shared[t] = the same with the shared expert on x[t].
 *   x          [T,d] (read only when n_shared == 1; may be NULL otherwise)
 *   x_perm     [R,d] act_dtype;  offsets [E+1] int32 (as moe_permute writes it)
 *   y_perm     [R,d] f32 out (rows >= offsets[E] untouched)
 *   y_shared   [T,d] f32 out, required iff n_shared == 1 */
moe_status moe_expert_ffn(const moe_config* cfg, const void* x, const void* x_perm,
                          const int32_t* offsets, const moe_expert_weights* weights,
                          float* y_perm, float* y_shared, void* ws, size_t ws_bytes,
                          void* stream);

/* Step 6: weighted combine ([P3] s3.1 output = sum of weight * expert output;
 * [P5] aggregation layer -- the residual add is left to the caller).
 *   out[t] = sum_{j: dest_row[t,j] >= 0} topk_w[t,j] * y_perm[dest_row[t,j]]
 *            (+ y_shared[t] when n_shared == 1), summed in j order in f32;
 *   out [T,d] out_dtype (bf16: one round-to-nearest-even at the end). */
moe_status moe_combine(const moe_config* cfg, const float* y_perm, const float* y_shared,
                       const int32_t* dest_row, const float* topk_w, void* out,
                       void* stream);

/* The whole layer ([P5] fused MoE forward: hidden states, router, experts ->
 * output).  Intermediates live in the workspace.
 *   stats    [2E+1] int32 out, or NULL: counts[E] (requested), kept[E] (final rows
 *            per expert, re-routed pairs included), n_dropped
 *   routing  optional copies of the routing decision, or NULL */
moe_status moe_forward(const moe_config* cfg, const void* x, const float* w_router,
                       const float* bias, const float* gumbel_u,
                       const moe_expert_weights* weights, void* out, int32_t* stats,
                       const moe_routing_out* routing, void* ws, size_t ws_bytes,
                       void* stream);

/* moe_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, results and errors as moe_forward
 * (bit-identical output), with the intermediates in a scratch array of
 * MOE_NOALLOC_SCRATCH_BYTES that the library's code object holds on every
 * device it is loaded on, until the process ends.  Nothing is allocated or
 * freed: the array's address is looked up once per device (the first call with
 * that device current) and reused.
 *   Limit: a layer whose moe_workspace_bytes exceeds MOE_NOALLOC_SCRATCH_BYTES
 *   is rejected with MOE_ERR_UNSUPPORTED before anything is launched (64 MiB
 *   covers decode and small batches: e.g. a Mixtral-shaped layer up to T = 256,
 *   the 256-expert fine-grained layer up to T = 128).
 *   Concurrency: every call on one device uses that device's one array, and the
 *   kernels need it from the first launch to the last; calls whose work
 *   overlaps on one device (other streams, other host threads) race and give
 *   wrong results.  Serialise them, or use moe_forward with one workspace each.
 *   The array keeps the last call's contents; no kernel relies on its initial
 *   contents. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_forward_noalloc(const moe_config* cfg, const void* x, const float* w_router,
                               const float* bias, const float* gumbel_u,
                               const moe_expert_weights* weights, void* out, int32_t* stats,
                               const moe_routing_out* routing, void* stream);

/* ---- load balancing after a routed batch ----
 * Mean router probability and the auxiliary-loss term ([P3] s4.3 training
 * stability: aux = sum_e mean_t(router_probs[t,e]) * expert_count[e]).  The
 * router probability of (t,e) is the distribution the gate weights are drawn
 * from before the top-k: the softmax over all E experts of the weight basis
 * (z, plus a logit bias, plus Gumbel noise, over tau) for softmax scoring, the
 * sigmoid scores normalised to sum 1 for sigmoid scoring; a selection-only
 * bias is not part of it.  Reduced in a fixed order in f64, rounded once.
 *   logits    [T,E] f32: the router logits of the batch (moe_route's or
 *             moe_forward's routing output)
 *   bias      [E] f32 as given to the routing call (read for a logit bias)
 *   gumbel_u  [T,E] f32 as given to the routing call, or NULL
 *   counts    [E] int32: pairs routed to each expert, before any capacity
 *             limit (moe_permute's counts; the first E entries of stats)
 *   prob_mean [E] f32 out: mean over the T tokens (0 when T == 0)
 *   aux       [1] f32 out, or NULL: sum_e prob_mean[e] * counts[e]
 *   ws        device workspace of at least moe_workspace_bytes(cfg) bytes */
moe_status moe_router_stats(const moe_config* cfg, const float* logits, const float* bias,
                            const float* gumbel_u, const int32_t* counts, float* prob_mean,
                            float* aux, void* ws, size_t ws_bytes, void* stream);

/* One loss-free balancing step of the per-expert bias ([P5] gating network:
 *   bias[e] <- decay * bias[e] - rate * counts[e] / (mean_e(counts) + 1e-8),
 * decay 0.99 and rate 0.01 in its routing configuration), in f64, rounded once.
 *   counts [E] int32 as for moe_router_stats;  bias [E] f32, updated in place.
 *   decay, rate: finite. */
moe_status moe_bias_update(const moe_config* cfg, const int32_t* counts, float* bias,
                           float decay, float rate, void* stream);

/* ---- measurement hooks (not part of the layer) ----
 * While enabled on the calling thread, every kernel the library launches is
 * bracketed by HIP events recorded on the launch stream.  moe_profile_read()
 * synchronises those events and returns, per kernel name, the launch count
 * and the summed duration in milliseconds, then clears the record. */
typedef struct {
  char name[48];
  int32_t launches;
  double total_ms;
} moe_kernel_time;

moe_status moe_profile_enable(int32_t on);
moe_status moe_profile_read(moe_kernel_time* out, int32_t max_entries, int32_t* n_entries);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
