"""Plant plausible mistakes in the oracle (CPU only) and check a pin catches each.

Every mutation replaces one oracle function with a subtly wrong version for
the duration of one test; the listed pin tests must then fail.  This is what
makes the pins in test_oracle_pins.py worth trusting.
"""
import math

import numpy as np
import pytest

from oracle import moe_oracle as O
import tests.test_oracle_pins as pins

_orig = {name: getattr(O, name) for name in
         ["router_logits", "gumbel_noise", "topk_by_keys", "gate_weights", "capacity",
          "permute", "swiglu_ffn", "combine", "fp8_e4m3fn_decode", "selection_keys",
          "silu", "router_probs", "router_stats", "bias_update", "permute_reroute",
          "group_limited_keys", "int4_dequant"]}


def m_router_wrong_column(x, w):
    return _orig["router_logits"](x, np.asarray(w)[:, ::-1])


def m_gumbel_sign(u):
    return (np.log(-np.log(np.asarray(u, np.float64)))).astype(np.float32)


def m_topk_ties_high(keys, k):
    keys = np.asarray(keys, np.float32)
    rev = keys[:, ::-1]
    idx, gs, go = _orig["topk_by_keys"](rev, k)
    return (keys.shape[1] - 1 - idx).astype(np.int32), gs, go


def m_weights_no_renorm(basis, idx, rc):
    rc2 = O.RouteConfig(rc.E, rc.k, rc.score, 0, rc.tau, rc.bias_mode)
    return _orig["gate_weights"](basis, idx, rc2)


def m_capacity_ceil(T, k, E, cf):
    if cf <= 0:
        return None
    return max(1, int(math.ceil(T * k * cf / E)))


def m_capacity_no_floor1(T, k, E, cf):
    if cf <= 0:
        return None
    return int(math.floor(T * k * cf / E))


def m_permute_keep_one_extra(idx, E, C):
    return _orig["permute"](idx, E, None if C is None else C + 1)


def m_swiglu_swapped(rows, wg, wu, wd):
    return _orig["swiglu_ffn"](rows, wu, wg, wd)


def m_swiglu_no_silu(rows, wg, wu, wd):
    r = np.asarray(rows, np.float64)
    return ((r @ wg.T) * (r @ wu.T)) @ wd.T


def m_combine_unweighted(y, dest, w, sh=None):
    return _orig["combine"](y, dest, np.ones_like(w), sh)


def m_fp8_bias8(codes):
    return _orig["fp8_e4m3fn_decode"](codes) / 2.0


def m_bias_in_weights(z, rc, bias=None, u=None):
    key, basis = _orig["selection_keys"](z, rc, bias, u)
    if rc.bias_mode == O.BIAS_SELECT_ONLY and rc.score == O.SCORE_SIGMOID:
        basis = key
    return key, basis


def _softmax_keys_variant(z, rc, bias, u, *, noise_tempered=True, logit_bias_tempered=True,
                          select_bias_tempered=False):
    """selection_keys for softmax scoring with the temperature placed elsewhere."""
    if rc.score != O.SCORE_SOFTMAX:
        return _orig["selection_keys"](z, rc, bias, u)
    f32 = np.float32
    z32 = np.asarray(z, f32)
    b32 = None if bias is None else np.asarray(bias, f32)[None, :]
    g = None if u is None else O.gumbel_noise(u)
    inner = z32.copy()
    if rc.bias_mode == O.BIAS_LOGIT and logit_bias_tempered:
        inner = (inner + b32).astype(f32)
    if g is not None and noise_tempered:
        inner = (inner + g).astype(f32)
    l = (inner / f32(rc.tau)).astype(f32)
    if rc.bias_mode == O.BIAS_LOGIT and not logit_bias_tempered:
        l = (l + b32).astype(f32)
    if g is not None and not noise_tempered:
        l = (l + g).astype(f32)
    key = l
    if rc.bias_mode == O.BIAS_SELECT_ONLY:
        key = (((l * f32(rc.tau)) + b32) / f32(rc.tau)).astype(f32) if select_bias_tempered else (l + b32).astype(f32)
    return key, l


def m_tau_divides_logit_only(z, rc, bias=None, u=None):
    """l = z / tau + g: the noise escapes the temperature."""
    return _softmax_keys_variant(z, rc, bias, u, noise_tempered=False)


def m_logit_bias_untempered(z, rc, bias=None, u=None):
    """l = (z + g) / tau + b: the logit bias escapes the temperature."""
    return _softmax_keys_variant(z, rc, bias, u, logit_bias_tempered=False)


def m_select_bias_tempered(z, rc, bias=None, u=None):
    """key = (z + g + b) / tau for a selection-only bias."""
    return _softmax_keys_variant(z, rc, bias, u, select_bias_tempered=True)


def m_probs_with_selection_bias(z, rc, bias=None, u=None):
    key, _ = O.selection_keys(z, rc, bias, u)
    k = np.asarray(key, np.float64)
    if rc.score == O.SCORE_SOFTMAX:
        ex = np.exp(k - k.max(axis=1, keepdims=True))
        return ex / ex.sum(axis=1, keepdims=True)
    return k / k.sum(axis=1, keepdims=True)


def m_probs_no_tau(z, rc, bias=None, u=None):
    rc1 = O.RouteConfig(rc.E, rc.k, rc.score, rc.renormalize, 1.0, rc.bias_mode)
    return _orig["router_probs"](z, rc1, bias, u)


def m_stats_sum_not_mean(probs, counts):
    P = np.asarray(probs, np.float64).sum(axis=0)
    return P, float(np.sum(P * np.asarray(counts, np.float64)))


def m_bias_wrong_sign(bias, counts, decay=0.99, rate=0.01):
    load = np.asarray(counts, np.float64)
    return (decay * np.asarray(bias, np.float64) + rate * load / (load.mean() + 1e-8)).astype(np.float32)


def m_bias_unnormalised_load(bias, counts, decay=0.99, rate=0.01):
    return (decay * np.asarray(bias, np.float64) - rate * np.asarray(counts, np.float64)).astype(np.float32)


def _reroute_variant(idx, fallback, E, C, *, check_load=True, distinct=True, reverse=False,
                     reroute_first=False):
    """The re-routing rule with one knob turned (a plausible mistake)."""
    idx = np.asarray(idx)
    fb = np.asarray(fallback)
    T, k = idx.shape
    if C is None:
        return _orig["permute"](idx, E, C)
    counts = np.bincount(idx.ravel(), minlength=E).astype(np.int64)
    kept1 = np.minimum(counts, C)
    rank1 = np.zeros((T, k), np.int64)
    seen = np.zeros(E, np.int64)
    for t in range(T):
        for j in range(k):
            rank1[t, j] = seen[idx[t, j]]
            seen[idx[t, j]] += 1
    load = kept1.copy()
    new_e = np.full((T, k), -1)
    rank2 = np.zeros((T, k), np.int64)
    order = range(T - 1, -1, -1) if reverse else range(T)
    for t in order:
        used = set()
        for j in range(k):
            if rank1[t, j] < C:
                continue
            for c in fb[t]:
                c = int(c)
                if (distinct and c in used) or (check_load and load[c] >= C):
                    continue
                new_e[t, j] = c
                rank2[t, j] = load[c] - kept1[c]
                load[c] += 1
                used.add(c)
                break
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(load)
    dest = np.full((T, k), -1, np.int64)
    src = np.full(max(T * k, int(load.sum())), -1, np.int64)
    for t in range(T):
        for j in range(k):
            if rank1[t, j] < C:
                e = idx[t, j]
                row = offsets[e] + rank1[t, j] + ((load[e] - kept1[e]) if reroute_first else 0)
            elif new_e[t, j] >= 0:
                c = new_e[t, j]
                row = offsets[c] + (0 if reroute_first else kept1[c]) + rank2[t, j]
            else:
                continue
            dest[t, j] = row
            src[row] = t
    return O.Permutation(counts.astype(np.int32), load.astype(np.int32), offsets.astype(np.int32),
                         dest.astype(np.int32), src[: T * k].astype(np.int32), int(T * k - load.sum()))


def m_reroute_ignores_capacity(idx, fb, E, C):
    return _reroute_variant(idx, fb, E, C, check_load=False)


def m_reroute_repeats_expert(idx, fb, E, C):
    return _reroute_variant(idx, fb, E, C, distinct=False)


def m_reroute_last_token_first(idx, fb, E, C):
    return _reroute_variant(idx, fb, E, C, reverse=True)


def m_reroute_rows_before_first_pass(idx, fb, E, C):
    return _reroute_variant(idx, fb, E, C, reroute_first=True)


def m_group_score_sum(keys, n_groups, topk_groups):
    keys = np.asarray(keys, np.float32)
    T, E = keys.shape
    gsz = E // n_groups
    gscore = keys.reshape(T, n_groups, gsz).astype(np.float64).sum(axis=2)
    order = np.argsort(-gscore, axis=1, kind="stable")
    keep = np.zeros((T, n_groups), bool)
    np.put_along_axis(keep, order[:, :topk_groups], True, axis=1)
    return np.where(np.repeat(keep, gsz, axis=1), keys, np.float32(-np.inf)).astype(np.float32), \
        np.full(T, np.inf)


def m_group_interleaved(keys, n_groups, topk_groups):
    keys = np.asarray(keys, np.float32)
    T, E = keys.shape
    perm = np.arange(E).reshape(E // n_groups, n_groups).T.ravel()  # group g = experts e with e % G == g
    lim, gap = _orig["group_limited_keys"](keys[:, perm], n_groups, topk_groups)
    out = np.empty_like(lim)
    out[:, perm] = lim
    return out, gap


def m_int4_nibbles_swapped(packed, qp):
    p = np.asarray(packed, np.uint8)
    return _orig["int4_dequant"]((p >> 4) | ((p & 15) << 4), qp)


def m_int4_zero_ignored(packed, qp):
    return _orig["int4_dequant"](packed, np.asarray(qp, np.uint32) & 0xFFFF)


def m_int4_groups_interleaved(packed, qp):
    """Group g of a row taken as columns g, g + G, g + 2G, ... instead of a block."""
    p = np.asarray(packed, np.uint8)
    q = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.int64)
    q[..., 0::2], q[..., 1::2] = p & 15, p >> 4
    qp = np.asarray(qp, np.uint32)
    s = (qp & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
    z = ((qp >> 16) & 15).astype(np.int64)
    reps = q.shape[-1] // qp.shape[-1]
    return np.tile(s, reps) * (q - np.tile(z, reps))


def m_int4_sign_flipped(packed, qp):
    return -_orig["int4_dequant"](packed, qp)


MUTATIONS = [
    ("router_logits", m_router_wrong_column, ["test_router_unit_vectors_select_rows"]),
    ("gumbel_noise", m_gumbel_sign, ["test_gumbel_statistics_match_gumbel01",
                                     "test_gumbel_noise_closed_form_points"]),
    ("topk_by_keys", m_topk_ties_high, ["test_topk_bruteforce_with_ties"]),
    ("gate_weights", m_weights_no_renorm, ["test_softmax_then_topk_equals_topk_then_softmax"]),
    ("capacity", m_capacity_ceil, ["test_capacity_worked_examples_from_pages"]),
    ("capacity", m_capacity_no_floor1, ["test_capacity_worked_examples_from_pages"]),
    ("permute", m_permute_keep_one_extra, ["test_forced_overflow_closed_form"]),
    ("swiglu_ffn", m_swiglu_swapped, ["test_single_expert_top1_is_dense_ffn"]),
    ("swiglu_ffn", m_swiglu_no_silu, ["test_single_expert_top1_is_dense_ffn",
                                      "test_swiglu_bruteforce_tiny"]),
    ("combine", m_combine_unweighted, ["test_identity_expert_combine_inverts_permute"]),
    ("fp8_e4m3fn_decode", m_fp8_bias8, ["test_fp8_decode_all_codes"]),
    ("selection_keys", m_bias_in_weights, ["test_selection_only_bias_steers_but_does_not_weigh"]),
    ("selection_keys", m_tau_divides_logit_only, ["test_temperature_divides_logit_plus_noise",
                                                  "test_logit_bias_noise_and_temperature_together"]),
    ("selection_keys", m_logit_bias_untempered, ["test_logit_bias_is_tempered_with_the_logit",
                                                 "test_logit_bias_noise_and_temperature_together"]),
    ("selection_keys", m_select_bias_tempered, ["test_selection_only_bias_is_added_after_the_temperature"]),
    ("router_probs", m_probs_with_selection_bias,
     ["test_router_probs_ignore_selection_only_bias_and_follow_logit_bias"]),
    ("router_probs", m_probs_no_tau, ["test_router_probs_are_the_unrenormalised_gate_weights"]),
    ("router_stats", m_stats_sum_not_mean, ["test_router_stats_hand_example_and_uniform_closed_form"]),
    ("bias_update", m_bias_wrong_sign, ["test_bias_update_hand_examples"]),
    ("bias_update", m_bias_unnormalised_load, ["test_bias_update_hand_examples"]),
    ("permute_reroute", m_reroute_ignores_capacity, ["test_reroute_hand_example_fills_next_best_free_expert"]),
    ("permute_reroute", m_reroute_repeats_expert,
     ["test_reroute_slots_of_one_token_take_distinct_experts_in_key_order"]),
    ("permute_reroute", m_reroute_last_token_first, ["test_reroute_priority_goes_to_the_earlier_token",
                                                     "test_reroute_matches_deferred_acceptance_bruteforce"]),
    ("permute_reroute", m_reroute_rows_before_first_pass, ["test_reroute_rows_follow_the_first_pass"]),
    ("group_limited_keys", m_group_score_sum, ["test_group_limit_hand_example", "test_group_limit_bruteforce"]),
    ("group_limited_keys", m_group_interleaved, ["test_group_limit_hand_example"]),
    ("int4_dequant", m_int4_nibbles_swapped, ["test_int4_hand_example", "test_int4_every_code_and_zero_point"]),
    ("int4_dequant", m_int4_zero_ignored, ["test_int4_hand_example", "test_int4_every_code_and_zero_point",
                                           "test_int4_groups_take_their_own_parameters"]),
    ("int4_dequant", m_int4_groups_interleaved, ["test_int4_groups_take_their_own_parameters"]),
    ("int4_dequant", m_int4_sign_flipped, ["test_int4_hand_example", "test_int4_every_code_and_zero_point"]),
]


@pytest.mark.parametrize("target,mutant,catchers", MUTATIONS,
                         ids=[m[1].__name__ for m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, target, mutant, catchers):
    monkeypatch.setattr(O, target, mutant)
    for name in catchers:
        fn = getattr(pins, name)
        with pytest.raises(AssertionError):
            fn()
