"""CPU oracle for the sparse MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and
its Python binding) never imports, calls or links anything under ``oracle/``,
and shares no code with it.

What it computes is the plain definition of the layer, step by step, in
float64 from the exact input values (bf16 and fp8 inputs widen exactly), with
float32 only where the layer's definition fixes float32:

* router logits z are float32 (the fp32 router of the Mixtral-shaped
  workload): the exact dot product rounded once;
* the selection keys are float32 values computed by float32 operations in a
  fixed order, because floating point decides an integer (the top-k) there
  and both implementations must take that decision in the same precision;
* gate weights are computed in float64 and rounded once to float32.

Sources (pages are cited by title, host and section; no line numbers):

[P1] "GPT-4 has 1.8T parameters but uses 2% per token: dynamic sparse
     activation" (mlqm.cn) -- s3.1 gating network (Gumbel noise, temperature
     0.5, softmax then top-2), s3.3 expert structure (SwiGLU FFN), s4.2 the
     sparse-MoE model code (router returns the top-k of the perturbed softmax
     as weights; weighted sum of expert outputs).
[P2] "Parameter scale and the truth about sparse activation" (deepseek.csdn.net)
     -- s3.1 top-k routing with temperature, s3.2 expert capacity formula and
     the "capacity >= 1" rule, s5.1 Gumbel jitter, s5.2 long-text capacity example.
[P3] "MoE sparse activation: principles and engineering practice"
     (kapook.pages.dev mirror of blog.csdn.net) -- s3.1 Router code (linear
     without bias, top-k sorted, softmax over the top-k logits, output is the
     weighted sum), s3.2 experts share one input/output shape.
[P4] "V4 full-stack architecture" (kwkr.cn) -- s2.2 fine-grained experts and
     an always-visited shared expert; the model config (256 experts, top-8).
[P5] "From sparse MoE to conditional memory" (m.nxbn.cn) -- "DeepSeek MoE
     dynamic routing" (per-expert bias steering the selection), "gating network
     implementation" (top-k on biased scores, softmax over the chosen).

Readings of points the pages leave open are listed beside the function that
takes them.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

SCORE_SOFTMAX, SCORE_SIGMOID = 0, 1
BIAS_NONE, BIAS_LOGIT, BIAS_SELECT_ONLY = 0, 1, 2
DT_F32, DT_BF16, DT_FP8 = 0, 1, 2


# ---------------------------------------------------------------------------
# S1 router
def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """z[t,e] = sum_i x[t,i] * W_r[i,e], rounded once to float32.

    [P3] s3.1 (router = linear layer d -> E without bias); [P1] s3.1 (a linear
    map from the d-dim token embedding to one logit per expert).  Inputs are
    float32 (bf16 values widen exactly); products and sums are float64.
    """
    x64 = np.asarray(x, dtype=np.float64)
    w64 = np.asarray(w_router, dtype=np.float64)
    return (x64 @ w64).astype(np.float32)


# ---------------------------------------------------------------------------
# S2 scores, selection keys, top-k, gate weights
def gumbel_noise(u: np.ndarray) -> np.ndarray:
    """g = -log(-log u) in float64, rounded to float32.  [P1] s3.1; [P2] s5.1."""
    u64 = np.asarray(u, dtype=np.float64)
    return (-np.log(-np.log(u64))).astype(np.float32)


def sigmoid_scores(z: np.ndarray) -> np.ndarray:
    """s = 1 / (1 + exp(-z)) in float64, rounded to float32.

    Sigmoid scoring is not on the pages; the fine-grained workload fixes it.
    """
    z64 = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return (1.0 / (1.0 + np.exp(-z64))).astype(np.float32)


@dataclasses.dataclass
class RouteConfig:
    E: int
    k: int
    score: int = SCORE_SOFTMAX
    renormalize: int = 1
    tau: float = 1.0
    bias_mode: int = BIAS_NONE
    n_groups: int = 0        # group-limited routing: experts in n_groups blocks (0/1 = off)
    topk_groups: int = 0     # groups kept per token


def selection_keys(z: np.ndarray, rc: RouteConfig, bias=None, u=None):
    """Return (keys, basis): float32 keys that decide the top-k, and the float32
    per-expert quantity the gate weights are computed from.

    softmax scoring  ([P1] s3.1, [P2] s3.1, [P5] gating network):
        l = z;  l = l + b   (logit bias);  l = l + g   (Gumbel);  l = l / tau
        key = l, or l + b for a selection-only bias; basis = l
    sigmoid scoring (fine-grained workload; bias steers selection only, as the
    per-expert bias of [P5] "DeepSeek MoE dynamic routing"):
        s = sigmoid(z);  key = s, or s + b;  basis = s
    Every arrow is one float32 operation, in this order.
    """
    z32 = np.asarray(z, dtype=np.float32)
    f32 = np.float32
    if bias is not None:
        b32 = np.asarray(bias, dtype=np.float32)[None, :]
    if rc.score == SCORE_SOFTMAX:
        l = z32.copy()
        if rc.bias_mode == BIAS_LOGIT:
            l = (l + b32).astype(f32)
        if u is not None:
            l = (l + gumbel_noise(u)).astype(f32)
        l = (l / f32(rc.tau)).astype(f32)
        key = l
        if rc.bias_mode == BIAS_SELECT_ONLY:
            key = (l + b32).astype(f32)
        return key, l
    if rc.score == SCORE_SIGMOID:
        if rc.bias_mode == BIAS_LOGIT or u is not None or rc.tau != 1.0:
            raise ValueError("sigmoid scoring takes no logit bias, noise or temperature")
        s = sigmoid_scores(z32)
        key = s
        if rc.bias_mode == BIAS_SELECT_ONLY:
            key = (s + b32).astype(f32)
        return key, s
    raise ValueError(rc.score)


def topk_by_keys(keys: np.ndarray, k: int):
    """Top-k of each row: descending key, ties to the lower expert index.

    [P3] s3.1 asks for the k largest, sorted; the tie rule is a reading
    of its own (torch leaves it open).  Uses a stable sort of -key as the library
    step.  Also returns, per token, the selection gap (k-th key minus the
    (k+1)-th) and the order gap (smallest difference between consecutive chosen
    keys), both in float64, so callers can set near-ties aside.
    """
    keys = np.asarray(keys, dtype=np.float32)
    T, E = keys.shape
    order = np.argsort(-keys.astype(np.float64), axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    ks = np.take_along_axis(keys.astype(np.float64), order, axis=1)
    gap_sel = ks[:, k - 1] - ks[:, k] if k < E else np.full(T, np.inf)
    if k > 1:
        gap_ord = np.min(ks[:, : k - 1] - ks[:, 1:k], axis=1)
    else:
        gap_ord = np.full(T, np.inf)
    return idx, gap_sel, gap_ord


def gate_weights(basis: np.ndarray, idx: np.ndarray, rc: RouteConfig) -> np.ndarray:
    """Gate weight of each chosen expert, float64 then rounded to float32.

    softmax, renormalised ([P3] s3.1 softmax over the top-k logits; equal to
      softmax-then-top-k renormalised to sum 1):
        w_j = exp(l_j - m) / sum_{j' chosen} exp(l_j' - m)
    softmax, not renormalised ([P1] s4.2 code: the weights are the top-k
      entries of the softmax over all E):
        w_j = exp(l_j - M) / sum_{e < E} exp(l_e - M)
    sigmoid: w_j = s_j / sum_{j' chosen} s_j'   (or s_j without renormalising)
    """
    b64 = np.asarray(basis, dtype=np.float64)
    chosen = np.take_along_axis(b64, idx.astype(np.int64), axis=1)
    if rc.score == SCORE_SOFTMAX:
        if rc.renormalize:
            m = chosen.max(axis=1, keepdims=True)
            ex = np.exp(chosen - m)
            w = ex / ex.sum(axis=1, keepdims=True)
        else:
            M = b64.max(axis=1, keepdims=True)
            w = np.exp(chosen - M) / np.exp(b64 - M).sum(axis=1, keepdims=True)
    else:
        w = chosen / chosen.sum(axis=1, keepdims=True) if rc.renormalize else chosen
    return w.astype(np.float32)


@dataclasses.dataclass
class Routing:
    idx: np.ndarray        # [T,k] int32
    w: np.ndarray          # [T,k] float32
    keys: np.ndarray       # [T,E] float32
    gap_sel: np.ndarray    # [T] float64
    gap_ord: np.ndarray    # [T] float64
    fallback: Optional[np.ndarray] = None  # [T,depth] int32 next-best experts, or None


def group_limited_keys(keys: np.ndarray, n_groups: int, topk_groups: int):
    """Two-level routing ([P3] closing case: experts clustered into groups, a
    router first decides the group, then the original router picks the experts
    inside it).  Reading: the experts form n_groups contiguous blocks of E /
    n_groups; a group's score is its largest key (the group holding the token's
    best expert comes first); the topk_groups best groups are kept, ties to the
    lower group; the other experts' keys become -inf so the top-k cannot take
    them.  Returns (limited keys float32, gap between the last kept and the first
    dropped group score, float64)."""
    keys = np.asarray(keys, np.float32)
    T, E = keys.shape
    gsz = E // n_groups
    gscore = keys.reshape(T, n_groups, gsz).max(axis=2).astype(np.float64)
    order = np.argsort(-gscore, axis=1, kind="stable")
    keep = np.zeros((T, n_groups), bool)
    np.put_along_axis(keep, order[:, :topk_groups], True, axis=1)
    srt = np.take_along_axis(gscore, order, axis=1)
    gap = srt[:, topk_groups - 1] - srt[:, topk_groups] if topk_groups < n_groups else np.full(T, np.inf)
    limited = np.where(np.repeat(keep, gsz, axis=1), keys, np.float32(-np.inf)).astype(np.float32)
    return limited, gap


def route_from_logits(z, rc: RouteConfig, bias=None, u=None, depth: int = 0) -> Routing:
    """S2 on given float32 logits: keys -> top-k -> gate weights (and the
    `depth` fallback experts for overflow re-routing).  With group-limited
    routing the top-k runs over the kept groups' experts only (the weights are
    formed as without it) and gap_sel also covers the group decision."""
    keys, basis = selection_keys(z, rc, bias, u)
    if rc.n_groups > 1:
        limited, ggap = group_limited_keys(keys, rc.n_groups, rc.topk_groups)
        idx, gs, go = topk_by_keys(limited, rc.k)
        gs = np.where(np.isfinite(gs), gs, np.inf)
        gs = np.minimum(gs, ggap)
        w = gate_weights(basis, idx, rc)
        fb = fallback_candidates(limited, rc.k, depth) if depth else None
        return Routing(idx, w, keys, gs, go, fb)
    idx, gs, go = topk_by_keys(keys, rc.k)
    w = gate_weights(basis, idx, rc)
    fb = fallback_candidates(keys, rc.k, depth) if depth else None
    return Routing(idx, w, keys, gs, go, fb)


# ---------------------------------------------------------------------------
# load-balancing statistics and the loss-free bias update (after the layer)
def router_probs(z, rc: RouteConfig, bias=None, u=None) -> np.ndarray:
    """Each token's probability of each expert, float64 [T, E].

    [P3] s4.3 (training stability, auxiliary loss) uses router_probs, every
    token's probability for every expert, without saying how it is formed.
    Reading: the distribution the gate weights are drawn from, before the top-k
    -- for softmax scoring the softmax over all E experts of the weight basis l
    (logit bias, Gumbel noise and temperature included, exactly as in the keys;
    a selection-only bias is not part of l), for sigmoid scoring the sigmoid
    scores normalised to sum 1 (the selection-only bias again left out).
    """
    _, basis = selection_keys(z, rc, bias, u)
    b = np.asarray(basis, np.float64)
    if rc.score == SCORE_SOFTMAX:
        ex = np.exp(b - b.max(axis=1, keepdims=True))
        return ex / ex.sum(axis=1, keepdims=True)
    return b / b.sum(axis=1, keepdims=True)


def router_stats(probs, counts):
    """Mean router probability per expert, and the auxiliary-loss term.

    [P3] s4.3: aux_loss = sum_e mean_t(router_probs[t, e]) * expert_count[e],
    expert_count[e] = how often expert e was chosen over all top-k slots (the
    requested counts, before any capacity limit).  The caller scales it (the
    page adds 0.01 * aux_loss to the main loss).  Returns (prob_mean [E]
    float64, aux float).
    """
    P = np.asarray(probs, np.float64).mean(axis=0)
    return P, float(np.sum(P * np.asarray(counts, np.float64)))


def bias_update(bias, counts, decay: float = 0.99, rate: float = 0.01) -> np.ndarray:
    """One loss-free balancing step on the per-expert selection bias, float32 [E].

    [P5] gating network code (balancing without an auxiliary loss): load[e] =
    how often expert e was chosen over all top-k slots; ratio = load /
    (mean(load) + 1e-8); bias <- decay * bias - rate * ratio, so busy experts'
    biases fall below idle ones'.  Its routing configuration sets decay 0.99
    and rate 0.01.  Computed in float64 and rounded once.
    """
    load = np.asarray(counts, np.float64)
    ratio = load / (load.mean() + 1e-8)
    return (float(decay) * np.asarray(bias, np.float64) - float(rate) * ratio).astype(np.float32)


# ---------------------------------------------------------------------------
# S3 capacity, counts, stable ranks; S4 permutation
def capacity(T: int, k: int, E: int, capacity_factor: float) -> Optional[int]:
    """C = max(1, floor(T * k / E * cf)); None (no limit) when cf <= 0.

    [P2] s3.2: capacity = tokens * k / experts * capacity_factor, and it must be
    at least 1.  The page's "1.2 -> 38 tokens (32 x 1.2)" example rounds 38.4
    down, so the reading is floor.  Evaluated in float64.
    """
    if capacity_factor <= 0:
        return None
    return max(1, int(math.floor(T * k * capacity_factor / E)))


@dataclasses.dataclass
class Permutation:
    counts: np.ndarray     # [E] int32: assignments per expert
    kept: np.ndarray       # [E] int32: min(counts, C)
    offsets: np.ndarray    # [E+1] int32: exclusive scan of kept
    dest_row: np.ndarray   # [T,k] int32: row in the permuted buffer, -1 = dropped
    src_token: np.ndarray  # [T*k] int32: token of each row, -1 past the kept rows
    n_dropped: int


def permute(idx: np.ndarray, E: int, C: Optional[int]) -> Permutation:
    """Counting sort of the (token, slot) pairs by expert, first come first kept.

    Pairs are visited in (t, j) order; a pair's rank is the number of earlier
    pairs routed to the same expert, and it is kept iff rank < C ([P2] s3.2:
    tokens over the limit are marked as overflow; a dropped pair contributes
    nothing -- no re-routing, no renormalisation).  Kept pairs of expert e take
    rows offsets[e] + rank, so each expert's rows are contiguous and in token
    order ([P3] s4.2 "expert fusion": one expert's tokens batched into one
    matmul; [P5] reorganising the tensor by routing index).
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    counts = np.zeros(E, dtype=np.int64)
    rank = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            rank[t, j] = counts[e]
            counts[e] += 1
    cap = np.iinfo(np.int64).max if C is None else C
    kept = np.minimum(counts, cap)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    dest = np.full((T, k), -1, dtype=np.int64)
    src = np.full(T * k, -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            if rank[t, j] < cap:
                row = offsets[idx[t, j]] + rank[t, j]
                dest[t, j] = row
                src[row] = t
    return Permutation(counts.astype(np.int32), kept.astype(np.int32),
                       offsets.astype(np.int32), dest.astype(np.int32),
                       src.astype(np.int32), int((counts - kept).sum()))


def fallback_candidates(keys: np.ndarray, k: int, depth: int) -> np.ndarray:
    """The `depth` next-best experts of each token after its top-k, by the same
    keys and tie rule as the top-k (int32 [T, depth])."""
    idx, _, _ = topk_by_keys(keys, k + depth)
    return idx[:, k:]


def permute_reroute(idx: np.ndarray, fallback: np.ndarray, E: int, C: Optional[int]) -> Permutation:
    """S3/S4 with the overflow re-routing of [P2] s3.2 ("Level 2": an overflowed
    token is not dropped; a fallback router takes its next-best expert that is
    not full).

    Reading, step by step:
      1. first pass exactly as permute(): pairs (t, j) ranked per expert in
         (t, j) order, kept iff rank < C;
      2. the pairs the first pass dropped are visited in the same (t, j) order;
         each takes the first expert of its token's fallback list (the next-best
         experts by key after the top-k, fallback_candidates) that holds fewer
         than C pairs at that moment and is not already serving the token
         through an earlier re-routed pair; if there is none it stays dropped;
      3. a re-routed pair keeps its gate weight (the weights are the routing's;
         only the expert serving the slot changes);
      4. expert e's rows are its first-pass pairs in (t, j) order, then its
         re-routed pairs in (t, j) order.
    counts stays the requested counts of the first pass; kept and offsets count
    the final rows; n_dropped the pairs left without an expert.
    """
    idx = np.asarray(idx)
    fb = np.asarray(fallback)
    T, k = idx.shape
    base = permute(idx, E, C)
    if C is None:
        return base
    counts = base.counts.astype(np.int64)
    kept1 = np.minimum(counts, C)
    rank1 = np.zeros((T, k), dtype=np.int64)
    seen = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            rank1[t, j] = seen[e]
            seen[e] += 1
    load = kept1.copy()
    new_e = np.full((T, k), -1, dtype=np.int64)
    rank2 = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        used = set()
        for j in range(k):
            if rank1[t, j] < C:
                continue
            for c in fb[t]:
                c = int(c)
                if c in used or load[c] >= C:
                    continue
                new_e[t, j] = c
                rank2[t, j] = load[c] - kept1[c]
                load[c] += 1
                used.add(c)
                break
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(load)
    dest = np.full((T, k), -1, dtype=np.int64)
    src = np.full(T * k, -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            if rank1[t, j] < C:
                row = offsets[idx[t, j]] + rank1[t, j]
            elif new_e[t, j] >= 0:
                c = new_e[t, j]
                row = offsets[c] + kept1[c] + rank2[t, j]
            else:
                continue
            dest[t, j] = row
            src[row] = t
    return Permutation(counts.astype(np.int32), load.astype(np.int32), offsets.astype(np.int32),
                       dest.astype(np.int32), src.astype(np.int32), int(T * k - load.sum()))


# ---------------------------------------------------------------------------
# S5/S6 expert FFN
def fp8_e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    """Decode OCP e4m3fn codes to float64 by the closed form.

    bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa:
      e > 0 : (-1)^s * 2^(e-7) * (1 + m/8)
      e = 0 : (-1)^s * 2^-6 * (m/8)
    S.1111.111 is NaN; there are no infinities (max 448).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 7), np.ldexp(m / 8.0, -6))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


INT4_GROUP = 128


def int4_dequant(packed, qparams) -> np.ndarray:
    """Group-wise INT4 expert weights to float64.

    [P3] s4.2 (quantisation and mixed precision): expert weights can be kept in
    INT4 while the router stays in higher precision, quantised group-wise --
    every 128 weights a group with its own scale and zero point.  Reading of the
    layout (the page gives none): groups run along each output row's input
    dimension; codes q in 0..15, two per byte, k = 2b in the low nibble of byte
    b and k = 2b + 1 in the high nibble ([..., N, K/2] uint8); per group one
    uint32, bits 0..15 the scale as IEEE fp16 and bits 16..19 the zero point z
    ([..., N, K/128]).  w[n, k] = scale * (q - z).
    """
    p = np.asarray(packed, dtype=np.uint8)
    q = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int64)
    q[..., 0::2] = p & 0xF
    q[..., 1::2] = p >> 4
    qp = np.asarray(qparams, dtype=np.uint32)
    scale = (qp & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
    zero = ((qp >> 16) & 0xF).astype(np.int64)
    return np.repeat(scale, INT4_GROUP, axis=-1) * (q - np.repeat(zero, INT4_GROUP, axis=-1))


def dequant(w, scale=None) -> np.ndarray:
    """Expert weight matrix to float64: widen f32/bf16, fp8 code * row scale, or
    group-wise INT4 (uint32 group parameters)."""
    w = np.asarray(w)
    if scale is not None and np.asarray(scale).dtype == np.uint32:
        return int4_dequant(w, scale)
    if w.dtype == np.uint8:
        return fp8_e4m3fn_decode(w) * np.asarray(scale, dtype=np.float64)[..., :, None]
    return w.astype(np.float64)


def silu(g: np.ndarray) -> np.ndarray:
    """silu(g) = g / (1 + exp(-g)) (the Swish-1 gate of SwiGLU)."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_ffn(rows: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """y = (silu(x Wg^T) * (x Wu^T)) Wd^T for row vectors x, in float64.

    [P1] s3.3 says the expert FFN uses SwiGLU (its code's two-matrix variant is
    a simplification); the standard three-matrix form with W_gate, W_up [F,d]
    and W_down [d,F] (stored [out, in]) is the reading.  No biases ([P1] s4.2
    and [P3] s3.1 use bias-free linear layers), no dropout ([P3] s3.2).
    """
    r = np.asarray(rows, dtype=np.float64)
    h = silu(r @ wg.T) * (r @ wu.T)
    return h @ wd.T


@dataclasses.dataclass
class ExpertWeights:
    """float64 views of the experts (dequantised on demand, one expert at a time)."""
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray
    s_gate: Optional[np.ndarray] = None
    s_up: Optional[np.ndarray] = None
    s_down: Optional[np.ndarray] = None

    def expert(self, e: int):
        sg = None if self.s_gate is None else self.s_gate[e]
        su = None if self.s_up is None else self.s_up[e]
        sd = None if self.s_down is None else self.s_down[e]
        return (dequant(self.w_gate[e], sg), dequant(self.w_up[e], su),
                dequant(self.w_down[e], sd))


def expert_outputs(x_perm: np.ndarray, offsets: np.ndarray, ew: ExpertWeights) -> np.ndarray:
    """y_perm[row] = SwiGLU_e(x_perm[row]) for the rows of each expert e."""
    E = len(offsets) - 1
    n = int(offsets[E])
    y = np.zeros((n, ew.w_down.shape[1]), dtype=np.float64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            wg, wu, wd = ew.expert(e)
            y[a:b] = swiglu_ffn(x_perm[a:b], wg, wu, wd)
    return y


# ---------------------------------------------------------------------------
# S7 combine
def combine(y_perm: np.ndarray, dest_row: np.ndarray, w: np.ndarray,
            y_shared: Optional[np.ndarray] = None) -> np.ndarray:
    """out[t] = sum_{j kept} w[t,j] * y_perm[dest_row[t,j]] (+ y_shared[t]).

    [P3] s3.1: the output is the weighted sum of the chosen experts' outputs;
    [P1] s4.2 weighted fusion; [P4] s2.2 the shared expert every token visits
    (reading: added with weight 1).  A token whose every pair was dropped gets
    zero (plus the shared output).  The residual add of [P5]'s aggregation
    layer is left to the caller.
    """
    T, k = dest_row.shape
    d = y_perm.shape[1] if y_perm.size else (y_shared.shape[1] if y_shared is not None else 0)
    out = np.zeros((T, d), dtype=np.float64)
    for j in range(k):
        keep = dest_row[:, j] >= 0
        rows = dest_row[keep, j]
        out[keep] += w[keep, j].astype(np.float64)[:, None] * y_perm[rows]
    if y_shared is not None:
        out += y_shared
    return out


# ---------------------------------------------------------------------------
# whole layer
@dataclasses.dataclass
class LayerSpec:
    T: int
    d: int
    E: int
    k: int
    F: int
    n_shared: int = 0
    score: int = SCORE_SOFTMAX
    renormalize: int = 1
    tau: float = 1.0
    bias_mode: int = BIAS_NONE
    capacity_factor: float = 0.0
    reroute_depth: int = 0
    n_groups: int = 0
    topk_groups: int = 0

    @property
    def route(self) -> RouteConfig:
        return RouteConfig(self.E, self.k, self.score, self.renormalize, self.tau, self.bias_mode,
                           self.n_groups, self.topk_groups)

    @property
    def C(self) -> Optional[int]:
        return capacity(self.T, self.k, self.E, self.capacity_factor)


@dataclasses.dataclass
class LayerResult:
    z: np.ndarray
    routing: Routing
    perm: Permutation
    x_perm: np.ndarray
    y_perm: np.ndarray
    y_shared: Optional[np.ndarray]
    out: np.ndarray


def forward(spec: LayerSpec, x, w_router, ew: ExpertWeights, shared: Optional[ExpertWeights] = None,
            bias=None, u=None, routing: Optional[Routing] = None) -> LayerResult:
    """The five steps in order: router, top-k, capacity + permutation, experts, combine.

    ``routing`` may be given to run S3..S7 on a routing decided elsewhere.
    """
    x64 = np.asarray(x, dtype=np.float64)
    z = router_logits(x, w_router)
    if routing is None:
        routing = route_from_logits(z, spec.route, bias, u, spec.reroute_depth)
    if spec.reroute_depth:
        perm = permute_reroute(routing.idx, routing.fallback, spec.E, spec.C)
    else:
        perm = permute(routing.idx, spec.E, spec.C)
    n = int(perm.offsets[spec.E])
    x_perm = x64[perm.src_token[:n]]
    y_perm = expert_outputs(x_perm, perm.offsets, ew)
    y_sh = None
    if spec.n_shared:
        wg, wu, wd = shared.expert(0)
        y_sh = swiglu_ffn(x64, wg, wu, wd)
    out = combine(y_perm, perm.dest_row, routing.w, y_sh)
    return LayerResult(z, routing, perm, x_perm, y_perm, y_sh, out)


def serving_experts(perm: Permutation) -> np.ndarray:
    """The expert whose rows hold each pair (-1 when dropped), from the offsets:
    the routed expert, or the fallback expert of a re-routed pair."""
    ex = np.searchsorted(perm.offsets, perm.dest_row, side="right") - 1
    return np.where(perm.dest_row >= 0, ex, -1).astype(np.int32)


def token_outputs(tokens, x, dest_row, idx, w, ew: ExpertWeights,
                  shared: Optional[ExpertWeights] = None) -> np.ndarray:
    """Layer output of selected tokens only, one by one, for a given routing.

    Same arithmetic as ``forward`` (expert FFN of the token's row, weighted sum,
    shared expert), organised per token so that single outputs of a large
    layer can be checked without running the whole layer on the CPU.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    x64 = np.asarray(x, dtype=np.float64)
    d = x64.shape[1]
    out = np.zeros((len(tokens), d), dtype=np.float64)
    needed = {}
    for i, t in enumerate(tokens):
        for j in range(idx.shape[1]):
            if dest_row[t, j] >= 0:
                needed.setdefault(int(idx[t, j]), []).append((i, j))
    for e, uses in sorted(needed.items()):
        wg, wu, wd = ew.expert(e)
        rows = np.stack([x64[tokens[i]] for i, _ in uses])
        y = swiglu_ffn(rows, wg, wu, wd)
        for (i, j), yr in zip(uses, y):
            out[i] += np.float64(w[tokens[i], j]) * yr
    if shared is not None:
        wg, wu, wd = shared.expert(0)
        out += swiglu_ffn(x64[tokens], wg, wu, wd)
    return out
