"""Pins of the CPU oracle against things other than itself (CPU only).

Each test checks one part of the oracle against a closed form, an invariant,
a special case that reduces to a library routine, brute force on a tiny
input, or a number the pages print (tests/golden/).  test_oracle_mutations.py
shows that plausible mistakes planted in the oracle fail at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- S1 router
def test_router_logits_match_exact_sum_bruteforce():
    """z = fl32(exact dot): math.fsum of exact float64 products (brute force)."""
    r = _rng(1)
    x = r.standard_normal((5, 37)).astype(np.float32)
    w = (0.02 * r.standard_normal((37, 3))).astype(np.float32)
    z = O.router_logits(x, w)
    for t in range(5):
        for e in range(3):
            exact = math.fsum(float(x[t, i]) * float(w[i, e]) for i in range(37))
            ref = np.float32(exact)
            # the float64 matmul may double-round: at most one float32 ulp away
            assert abs(float(z[t, e]) - float(ref)) <= float(np.spacing(np.float32(abs(ref))))


def test_router_unit_vectors_select_rows():
    """Closed form: x = e_i gives z = W_r[i, :] exactly; E = 1 gives a column dot."""
    r = _rng(2)
    w = r.standard_normal((6, 4)).astype(np.float32)
    z = O.router_logits(np.eye(6, dtype=np.float32), w)
    assert np.array_equal(z, w)
    w1 = r.standard_normal((6, 1)).astype(np.float32)
    x = r.standard_normal((3, 6)).astype(np.float32)
    z1 = O.router_logits(x, w1)
    assert z1.shape == (3, 1)


# ---------------------------------------------------------------- S2 top-k
def test_topk_bruteforce_with_ties():
    """Top-k equals Python's sort by (-key, expert); ties go to the lower index."""
    r = _rng(3)
    keys = r.integers(-3, 4, size=(200, 7)).astype(np.float32)  # many exact ties
    for k in (1, 2, 3, 7):
        idx, gs, go = O.topk_by_keys(keys, k)
        for t in range(200):
            ref = sorted(range(7), key=lambda e: (-float(keys[t, e]), e))[:k]
            assert list(idx[t]) == ref
            # the chosen set dominates the rest
            chosen = set(ref)
            rest = [e for e in range(7) if e not in chosen]
            if rest:
                assert min(keys[t, list(chosen)]) >= max(keys[t, rest])


def test_topk_subset_bruteforce():
    """The chosen set maximises the key sum over all k-subsets (distinct keys)."""
    r = _rng(4)
    keys = r.standard_normal((50, 6)).astype(np.float32)
    idx, _, _ = O.topk_by_keys(keys, 3)
    for t in range(50):
        best = max(itertools.combinations(range(6), 3), key=lambda s: sum(float(keys[t, e]) for e in s))
        assert set(idx[t]) == set(best)
        # descending order of the chosen keys
        assert all(keys[t, idx[t, j]] >= keys[t, idx[t, j + 1]] for j in range(2))


def test_gaps():
    keys = np.array([[5.0, 1.0, 3.0, 3.0, 0.5]], dtype=np.float32)
    idx, gs, go = O.topk_by_keys(keys, 3)
    assert list(idx[0]) == [0, 2, 3]
    assert gs[0] == pytest.approx(2.0)        # 3 - 1
    assert go[0] == 0.0                       # 3 - 3 is an order near-tie


def test_softmax_then_topk_equals_topk_then_softmax():
    """Identity: renormalised softmax-then-top-k (page P1's order) equals softmax over
    the top-k logits (page P3's code), computed here with torch.softmax."""
    r = _rng(5)
    z = (3 * r.standard_normal((100, 16))).astype(np.float32)
    rc = O.RouteConfig(E=16, k=4)
    route = O.route_from_logits(z, rc)
    probs = torch.softmax(torch.from_numpy(z.astype(np.float64)), dim=-1)
    top = torch.topk(probs, 4, dim=-1)
    ren = (top.values / top.values.sum(-1, keepdim=True)).numpy()
    assert np.array_equal(top.indices.numpy(), route.idx)
    np.testing.assert_allclose(route.w, ren, rtol=1e-6, atol=1e-7)


def test_k_equals_E_gives_full_softmax():
    r = _rng(6)
    z = r.standard_normal((20, 8)).astype(np.float32)
    for renorm in (0, 1):
        rc = O.RouteConfig(E=8, k=8, renormalize=renorm)
        route = O.route_from_logits(z, rc)
        full = torch.softmax(torch.from_numpy(z.astype(np.float64)), -1).numpy()
        got = np.zeros_like(full)
        np.put_along_axis(got, route.idx.astype(np.int64), route.w.astype(np.float64), axis=1)
        np.testing.assert_allclose(got, full, rtol=1e-6, atol=1e-8)
        np.testing.assert_allclose(route.w.sum(1), 1.0, rtol=1e-6)


def test_no_renormalisation_takes_topk_of_full_softmax():
    """Page P1's router code: weights are the top-k entries of softmax over all E."""
    r = _rng(7)
    z = r.standard_normal((30, 16)).astype(np.float32)
    rc = O.RouteConfig(E=16, k=2, renormalize=0, tau=0.5)
    route = O.route_from_logits(z, rc)
    full = torch.softmax(torch.from_numpy(z.astype(np.float64)) / 0.5, -1)
    top = torch.topk(full, 2, -1)
    assert np.array_equal(top.indices.numpy(), route.idx)
    np.testing.assert_allclose(route.w, top.values.numpy(), rtol=1e-6)


def test_gumbel_noise_closed_form_points():
    """g(u) = -log(-log u): u = exp(-exp(-c)) gives c; u = 1/e gives 0."""
    cs = np.array([-2.0, -0.5, 0.0, 0.7, 3.0], dtype=np.float64)
    u = np.exp(-np.exp(-cs)).astype(np.float32)
    g = O.gumbel_noise(u).astype(np.float64)
    # u was rounded to float32: error propagates as |dg/du| * ulp(u)
    du = np.abs(u.astype(np.float64) - np.exp(-np.exp(-cs)))
    slope = 1.0 / (np.exp(-np.exp(-cs)) * np.exp(-cs))
    assert np.all(np.abs(g - cs) <= slope * du + 1e-6)
    assert abs(float(O.gumbel_noise(np.array([np.exp(-1)], np.float32))[0])) < 1e-7


def test_gumbel_statistics_match_gumbel01():
    """Mean of Gumbel(0,1) is the Euler-Mascheroni constant, variance pi^2/6; a
    sign slip (Gumbel-min) flips the mean."""
    from mixture_experts_sparse_amd import workloads as W
    sh = W.WORKLOADS["gumbel_bf16"].replace(T=20000, E=16)
    g = O.gumbel_noise(W.gumbel_uniforms(sh)).astype(np.float64).ravel()
    assert abs(g.mean() - 0.5772156649) < 0.01
    assert abs(g.var() - math.pi ** 2 / 6) < 0.03


def test_gumbel_max_trick_samples_softmax():
    """argmax(z + g) is distributed as softmax(z) (the Gumbel-max property)."""
    r = _rng(8)
    z = np.array([0.3, -0.2, 1.1, 0.0], dtype=np.float32)
    n = 40000
    m = r.integers(0, 1 << 23, size=(n, 4))
    u = ((m + 0.5) * 2.0 ** -23).astype(np.float32)
    rc = O.RouteConfig(E=4, k=1, tau=1.0)
    route = O.route_from_logits(np.tile(z, (n, 1)), rc, u=u)
    freq = np.bincount(route.idx[:, 0], minlength=4) / n
    p = torch.softmax(torch.from_numpy(z.astype(np.float64)), -1).numpy()
    assert np.all(np.abs(freq - p) < 0.01)


def test_gumbel_zero_noise_reduces_to_tempered_softmax():
    r = _rng(9)
    z = r.standard_normal((64, 16)).astype(np.float32)
    u = np.full((64, 16), np.float32(np.exp(-1.0)), dtype=np.float32)
    rc = O.RouteConfig(E=16, k=2, tau=0.5, renormalize=0)
    a = O.route_from_logits(z, rc, u=u)
    b = O.route_from_logits(z, rc)
    clear = b.gap_sel > 1e-5
    assert np.array_equal(a.idx[clear], b.idx[clear])
    np.testing.assert_allclose(a.w, b.w, rtol=1e-5)


def test_sigmoid_selection_and_bias_invariance():
    r = _rng(10)
    z = r.standard_normal((100, 32)).astype(np.float32)
    rc = O.RouteConfig(E=32, k=4, score=O.SCORE_SIGMOID, bias_mode=O.BIAS_SELECT_ONLY)
    # constant bias: top-k of sigmoid(z) + c is the top-k of z (monotone)
    a = O.route_from_logits(z, rc, bias=np.full(32, 0.25, np.float32))
    idx_z, gs, _ = O.topk_by_keys(z, 4)
    clear = gs > 1e-3
    assert np.array_equal(a.idx[clear], idx_z[clear])
    # weights are the unbiased sigmoid normalised over the chosen experts
    s = 1.0 / (1.0 + np.exp(-z.astype(np.float64)))
    ch = np.take_along_axis(s, a.idx.astype(np.int64), 1)
    np.testing.assert_allclose(a.w, ch / ch.sum(1, keepdims=True), rtol=1e-6)
    # a bias that changes nothing in the selection changes nothing in the weights
    b = O.route_from_logits(z, rc, bias=np.zeros(32, np.float32))
    same = np.all(a.idx == b.idx, axis=1)
    np.testing.assert_array_equal(a.w[same], b.w[same])
    assert float(O.sigmoid_scores(np.zeros(1, np.float32))[0]) == 0.5


def test_selection_only_bias_steers_but_does_not_weigh():
    z = np.array([[0.0, 0.1, 0.2, 0.3]], dtype=np.float32)
    rc = O.RouteConfig(E=4, k=2, score=O.SCORE_SIGMOID, bias_mode=O.BIAS_SELECT_ONLY)
    route = O.route_from_logits(z, rc, bias=np.array([5.0, 4.0, 0.0, 0.0], np.float32))
    assert list(route.idx[0]) == [0, 1]
    s0, s1 = 0.5, 1 / (1 + math.exp(-0.1))
    np.testing.assert_allclose(route.w[0], [s0 / (s0 + s1), s1 / (s0 + s1)], rtol=1e-6)


def test_logit_bias_enters_softmax():
    z = np.zeros((1, 3), dtype=np.float32)
    b = np.array([0.0, math.log(3.0), -10.0], np.float32)
    rc = O.RouteConfig(E=3, k=2, bias_mode=O.BIAS_LOGIT)
    route = O.route_from_logits(z, rc, bias=b)
    assert list(route.idx[0]) == [1, 0]
    np.testing.assert_allclose(route.w[0], [0.75, 0.25], rtol=1e-6)


def _uniform_for_noise(c):
    """u = exp(-exp(-c)) as float32, so that -log(-log u) = c up to the rounding
    of u; returns u and a bound on |g - c| from that rounding."""
    c = np.asarray(c, np.float64)
    u64 = np.exp(-np.exp(-c))
    u = u64.astype(np.float32)
    slope = 1.0 / (u64 * np.exp(-c))          # |dg/du| at u
    return u, float(np.max(slope * np.abs(u.astype(np.float64) - u64))) + 1e-7


def test_temperature_divides_logit_plus_noise():
    """Page P1 (mlqm.cn) s3.1: the perturbed logits are (z + g) / tau, then the
    softmax.  Hand case, tau = 0.5, Gumbel noise fixed to known values:
    z = (0, 1, 0, 0), g = (1.2, 0, 0.9, 0) -> l = (2.4, 2.0, 1.8, 0).  The top-2
    is (0, 1) in that order, and without renormalisation (the Gumbel workload)
    the weights are e^2.4 / S and e^2.0 / S with S = e^2.4 + e^2 + e^1.8 + 1.
    Dividing only z by tau (z / tau + g = (1.2, 2.0, 0.9, 0)) reverses the order."""
    z = np.array([[0.0, 1.0, 0.0, 0.0]], np.float32)
    u, gerr = _uniform_for_noise([[1.2, 0.0, 0.9, 0.0]])
    rc = O.RouteConfig(E=4, k=2, tau=0.5, renormalize=0)
    route = O.route_from_logits(z, rc, u=u)
    assert list(route.idx[0]) == [0, 1]
    S = math.exp(2.4) + math.exp(2.0) + math.exp(1.8) + 1.0
    # each l moves by at most 2 gerr (1/tau), so each weight by about 4 gerr relative
    np.testing.assert_allclose(route.w[0], [math.exp(2.4) / S, math.exp(2.0) / S], rtol=8 * gerr + 1e-6)
    np.testing.assert_allclose(route.keys[0], [2.4, 2.0, 1.8, 0.0], atol=4 * gerr + 1e-6)
    # renormalised over the chosen two: e^0.4 / (e^0.4 + 1)
    rc1 = O.RouteConfig(E=4, k=2, tau=0.5, renormalize=1)
    w1 = O.route_from_logits(z, rc1, u=u).w[0]
    p = math.exp(0.4) / (math.exp(0.4) + 1.0)
    np.testing.assert_allclose(w1, [p, 1.0 - p], rtol=8 * gerr + 1e-6)


def test_logit_bias_is_tempered_with_the_logit():
    """A logit bias is part of the logit, so the temperature divides it too:
    l = (z + b) / tau.  z = 0, b = (0, ln 3, -10), tau = 0.5 -> l = (0, 2 ln 3,
    -20): the top-2 is (1, 0) with renormalised weights 9/10, 1/10 (a bias added
    after the temperature would give 3/4, 1/4)."""
    z = np.zeros((1, 3), dtype=np.float32)
    b = np.array([0.0, math.log(3.0), -10.0], np.float32)
    rc = O.RouteConfig(E=3, k=2, tau=0.5, bias_mode=O.BIAS_LOGIT)
    route = O.route_from_logits(z, rc, bias=b)
    assert list(route.idx[0]) == [1, 0]
    np.testing.assert_allclose(route.w[0], [0.9, 0.1], rtol=1e-6)


def test_logit_bias_noise_and_temperature_together():
    """All three at once: l = (z + b + g) / tau.  z = (0.5, 0, 0), b = (0, 0.25,
    0), g = (0, 0.5, -0.5), tau = 0.25 -> l = (2, 3, -2); renormalised top-2 is
    (1, 0) with weights e / (e + 1), 1 / (e + 1)."""
    z = np.array([[0.5, 0.0, 0.0]], np.float32)
    b = np.array([0.0, 0.25, 0.0], np.float32)
    u, gerr = _uniform_for_noise([[0.0, 0.5, -0.5]])
    rc = O.RouteConfig(E=3, k=2, tau=0.25, bias_mode=O.BIAS_LOGIT)
    route = O.route_from_logits(z, rc, bias=b, u=u)
    assert list(route.idx[0]) == [1, 0]
    p = math.e / (math.e + 1.0)
    np.testing.assert_allclose(route.w[0], [p, 1.0 - p], rtol=16 * gerr + 1e-6)
    np.testing.assert_allclose(route.keys[0], [2.0, 3.0, -2.0], atol=8 * gerr + 1e-6)


def test_selection_only_bias_is_added_after_the_temperature():
    """With softmax scoring, a selection-only bias steers the choice and is not
    part of the logit: key = (z + g) / tau + b, weights from (z + g) / tau.
    z = (0, 1, 0.5), tau = 0.5, b = (1.5, 0, 0): l = (0, 2, 1), keys = (1.5, 2, 1):
    the top-2 is (1, 0) and the renormalised weights are e^2 / (e^2 + 1), 1 / (e^2 + 1).
    A bias divided by tau as well (keys (3, 2, 1)) puts expert 0 first."""
    z = np.array([[0.0, 1.0, 0.5]], np.float32)
    b = np.array([1.5, 0.0, 0.0], np.float32)
    rc = O.RouteConfig(E=3, k=2, tau=0.5, bias_mode=O.BIAS_SELECT_ONLY)
    route = O.route_from_logits(z, rc, bias=b)
    assert list(route.idx[0]) == [1, 0]
    e2 = math.exp(2.0)
    np.testing.assert_allclose(route.w[0], [e2 / (e2 + 1.0), 1.0 / (e2 + 1.0)], rtol=1e-6)


# ---------------------------------------------------------------- S3 capacity
def test_capacity_worked_examples_from_pages():
    with open(os.path.join(GOLDEN, "capacity_examples.json")) as f:
        ex = json.load(f)["examples"]
    for e in ex:
        raw = e["tokens"] * e["k"] / e["experts"] * e["capacity_factor"]
        assert raw == pytest.approx(e["raw"])
        assert O.capacity(e["tokens"], e["k"], e["experts"], e["capacity_factor"]) == e["capacity"]


def test_capacity_of_the_skewed_workload():
    assert O.capacity(16384, 2, 128, 1.25) == 320
    assert O.capacity(32, 2, 128, 1.25) == 1
    assert O.capacity(64, 2, 8, 0.0) is None


def _brute_permute(idx, E, C):
    """Independent formulation: per-expert lists of pairs in (t, j) order, truncated."""
    T, k = idx.shape
    lists = [[] for _ in range(E)]
    for t in range(T):
        for j in range(k):
            lists[idx[t, j]].append((t, j))
    rows, dest = [], {}
    for e in range(E):
        keep = lists[e] if C is None else lists[e][:C]
        for p in keep:
            dest[p] = len(rows)
            rows.append(p[0])
    return lists, rows, dest


@pytest.mark.parametrize("C", [None, 1, 3, 17])
def test_permute_invariants_and_bruteforce(C):
    r = _rng(11)
    T, k, E = 97, 3, 9
    idx = np.stack([r.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    P = O.permute(idx, E, C)
    lists, rows, dest = _brute_permute(idx, E, C)
    assert P.counts.sum() == T * k
    assert P.kept.sum() + P.n_dropped == T * k
    assert list(P.counts) == [len(l) for l in lists]
    if C is not None:
        assert P.kept.max() <= C
    assert P.offsets[0] == 0 and np.all(np.diff(P.offsets) >= 0) and P.offsets[-1] == P.kept.sum()
    n = int(P.offsets[-1])
    assert list(P.src_token[:n]) == rows and np.all(P.src_token[n:] == -1)
    for t in range(T):
        for j in range(k):
            assert P.dest_row[t, j] == dest.get((t, j), -1)
    # bijection from kept pairs onto rows 0..n-1
    kept_rows = P.dest_row[P.dest_row >= 0]
    assert sorted(kept_rows.tolist()) == list(range(n))
    # inside each expert segment, tokens ascend
    for e in range(E):
        seg = P.src_token[P.offsets[e]:P.offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)


def test_forced_overflow_closed_form():
    """Every token sent to one expert with k = 1: exactly T - C dropped."""
    T, E = 200, 16
    for cf in (0.5, 1.0, 1.25, 3.0):
        C = O.capacity(T, 1, E, cf)
        idx = np.full((T, 1), 5, dtype=np.int32)
        P = O.permute(idx, E, C)
        assert P.n_dropped == T - min(T, C)
        assert P.kept[5] == min(T, C)
        # the first C tokens are the kept ones
        assert np.all(P.dest_row[:C, 0] == np.arange(C)) and np.all(P.dest_row[C:, 0] == -1)


def test_permutation_independent_of_slot_order():
    """Rows depend on which experts a token chose, not on the order of its k slots."""
    r = _rng(12)
    idx = np.stack([r.choice(6, 2, replace=False) for _ in range(40)]).astype(np.int32)
    a = O.permute(idx, 6, None)
    b = O.permute(idx[:, ::-1].copy(), 6, None)
    assert np.array_equal(a.src_token, b.src_token)
    assert np.array_equal(a.dest_row, b.dest_row[:, ::-1])


# ---------------------------------------------------------------- fp8
def test_fp8_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    dec = O.fp8_e4m3fn_decode(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(dec), nan) and nan.sum() == 2
    assert np.array_equal(dec[~nan], lib[~nan])
    assert dec[0x7E] == 448.0 and dec[0x38] == 1.0 and dec[0x01] == 2.0 ** -9 and dec[0x08] == 2.0 ** -6
    assert dec[0x80] == 0.0 and dec[0xFE] == -448.0


# ---------------------------------------------------------------- INT4 groups
def _qp(scale_bits, zero):
    return np.uint32(scale_bits | (zero << 16))


def test_int4_hand_example():
    """[P3] s4.2 group-wise INT4: one 128-wide group, scale 0.5 (fp16 0x3800),
    zero point 1.  Byte 0 = 0x21 holds codes 1 (k=0, low nibble) and 2 (k=1),
    byte 1 = 0xF0 holds 0 and 15; the rest 0x11 (code 1, value 0)."""
    row = np.full((1, 64), 0x11, np.uint8)
    row[0, 0], row[0, 1] = 0x21, 0xF0
    w = O.int4_dequant(row, np.array([[_qp(0x3800, 1)]], np.uint32))
    assert w.shape == (1, 128)
    np.testing.assert_array_equal(w[0, :4], [0.0, 0.5, -0.5, 7.0])
    assert np.all(w[0, 4:] == 0.0)


def test_int4_every_code_and_zero_point():
    """Scale 1 (fp16 0x3C00): byte b decodes to (b & 15) - z at k = 2b and
    (b >> 4) - z at k = 2b + 1, for all 256 bytes and all 16 zero points."""
    packed = np.tile(np.arange(256, dtype=np.uint8), (16, 1))   # K = 512: four groups
    qp = np.array([[_qp(0x3C00, z)] * 4 for z in range(16)], np.uint32)
    w = O.int4_dequant(packed, qp)
    b = np.arange(256)
    for z in range(16):
        assert np.array_equal(w[z, 0::2], (b & 15) - z)
        assert np.array_equal(w[z, 1::2], (b >> 4) - z)


def test_int4_groups_take_their_own_parameters():
    """Two groups per row, two rows: columns 0..127 use the row's first word,
    128..255 the second; fp16 scale bits decode by the IEEE formula
    2^(e-15) (1 + m/1024) for normal numbers and m 2^-24 for subnormal ones."""
    def f16(bits):
        e, m = (bits >> 10) & 31, bits & 1023
        v = m * 2.0 ** -24 if e == 0 else 2.0 ** (e - 15) * (1 + m / 1024)
        return -v if bits & 0x8000 else v
    packed = np.full((2, 128), 0x77, np.uint8)  # every code 7
    bits = [[0x4000, 0x3555], [0x0003, 0x7BFF]]
    zeros = [[3, 9], [0, 15]]
    qp = np.array([[_qp(bits[r][g], zeros[r][g]) for g in range(2)] for r in range(2)], np.uint32)
    w = O.int4_dequant(packed, qp)
    for r in range(2):
        for g in range(2):
            assert np.all(w[r, 128 * g:128 * (g + 1)] == f16(bits[r][g]) * (7 - zeros[r][g])), (r, g)


def test_int4_expert_dequant_dispatches_on_group_words():
    """dequant() takes the INT4 path for uint32 group words, fp8 for float scales."""
    packed = np.full((3, 64), 0x98, np.uint8)   # codes 8, 9
    w = O.dequant(packed, np.full((3, 1), _qp(0x3C00, 8), np.uint32))
    assert w.shape == (3, 128) and np.all(w[:, 0::2] == 0.0) and np.all(w[:, 1::2] == 1.0)


# ---------------------------------------------------------------- S5/S6 experts
def _dense_ffn_torch(x, wg, wu, wd):
    """SwiGLU from torch's library routines (linear, silu) in float64."""
    X = torch.from_numpy(np.asarray(x, np.float64))
    g = torch.nn.functional.linear(X, torch.from_numpy(wg))
    u = torch.nn.functional.linear(X, torch.from_numpy(wu))
    return torch.nn.functional.linear(torch.nn.functional.silu(g) * u, torch.from_numpy(wd)).numpy()


def _rand_experts(r, E, d, F):
    return O.ExpertWeights((0.2 * r.standard_normal((E, F, d))),
                           (0.2 * r.standard_normal((E, F, d))),
                           (0.2 * r.standard_normal((E, d, F))))


def test_single_expert_top1_is_dense_ffn():
    r = _rng(13)
    T, d, F = 33, 12, 20
    x = r.standard_normal((T, d)).astype(np.float32)
    ew = _rand_experts(r, 1, d, F)
    spec = O.LayerSpec(T, d, 1, 1, F)
    res = O.forward(spec, x, r.standard_normal((d, 1)).astype(np.float32), ew)
    ref = _dense_ffn_torch(x, ew.w_gate[0], ew.w_up[0], ew.w_down[0])
    np.testing.assert_allclose(res.out, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("renorm", [1, 0])
def test_identical_experts_reproduce_dense_ffn(renorm):
    r = _rng(14)
    T, d, F, E, k = 40, 10, 14, 6, 3
    x = r.standard_normal((T, d)).astype(np.float32)
    one = _rand_experts(r, 1, d, F)
    ew = O.ExpertWeights(np.repeat(one.w_gate, E, 0), np.repeat(one.w_up, E, 0),
                         np.repeat(one.w_down, E, 0))
    spec = O.LayerSpec(T, d, E, k, F, renormalize=renorm)
    res = O.forward(spec, x, r.standard_normal((d, E)).astype(np.float32), ew)
    ref = _dense_ffn_torch(x, one.w_gate[0], one.w_up[0], one.w_down[0])
    scale = res.routing.w.astype(np.float64).sum(1, keepdims=True)
    if renorm:
        np.testing.assert_allclose(scale, 1.0, rtol=1e-6)
    np.testing.assert_allclose(res.out, scale * ref, rtol=1e-10, atol=1e-12)


def test_grouped_experts_match_per_expert_dense():
    """Each expert's rows of y_perm equal that expert's dense FFN (with d != F,
    so a transposed operand cannot pass)."""
    r = _rng(15)
    T, d, F, E, k = 50, 8, 13, 5, 2
    x = r.standard_normal((T, d)).astype(np.float32)
    ew = _rand_experts(r, E, d, F)
    spec = O.LayerSpec(T, d, E, k, F)
    res = O.forward(spec, x, r.standard_normal((d, E)).astype(np.float32), ew)
    for e in range(E):
        a, b = res.perm.offsets[e], res.perm.offsets[e + 1]
        toks = res.perm.src_token[a:b]
        ref = _dense_ffn_torch(x[toks], ew.w_gate[e], ew.w_up[e], ew.w_down[e])
        np.testing.assert_allclose(res.y_perm[a:b], ref, rtol=1e-12, atol=1e-12)


def test_swiglu_bruteforce_tiny():
    """Scalar loops with math.exp on a 2x3 -> 4 -> 3 case."""
    r = _rng(16)
    x = r.standard_normal((2, 3))
    wg, wu, wd = r.standard_normal((4, 3)), r.standard_normal((4, 3)), r.standard_normal((3, 4))
    y = O.swiglu_ffn(x, wg, wu, wd)
    for t in range(2):
        h = []
        for f in range(4):
            g = sum(x[t, i] * wg[f, i] for i in range(3))
            u = sum(x[t, i] * wu[f, i] for i in range(3))
            h.append(g / (1 + math.exp(-g)) * u)
        for o in range(3):
            assert y[t, o] == pytest.approx(sum(h[f] * wd[o, f] for f in range(4)), rel=1e-12)


def test_fp8_expert_dequant_uses_row_scales():
    codes = np.array([[0x38, 0xB8], [0x40, 0x30]], dtype=np.uint8)  # 1, -1 ; 2, 0.5
    w = O.dequant(codes, np.array([0.5, 3.0]))
    np.testing.assert_array_equal(w, [[0.5, -0.5], [6.0, 1.5]])


# ---------------------------------------------------------------- S7 combine
def test_identity_expert_combine_inverts_permute():
    """With y := x_perm, renormalised weights and no drops, combine(permute(x)) = x."""
    r = _rng(17)
    T, d, E, k = 70, 9, 7, 3
    x = r.standard_normal((T, d))
    z = r.standard_normal((T, E)).astype(np.float32)
    route = O.route_from_logits(z, O.RouteConfig(E, k))
    P = O.permute(route.idx, E, None)
    xp = x[P.src_token[:P.offsets[-1]]]
    out = O.combine(xp, P.dest_row, route.w)
    np.testing.assert_allclose(out, x * route.w.astype(np.float64).sum(1, keepdims=True), rtol=1e-12)
    np.testing.assert_allclose(out, x, rtol=1e-6, atol=1e-6)


def test_dropped_tokens_get_zero_plus_shared():
    T, d, E = 12, 4, 3
    idx = np.zeros((T, 1), dtype=np.int32)
    w = np.ones((T, 1), dtype=np.float32)
    P = O.permute(idx, E, 5)
    y = np.arange(5 * d, dtype=np.float64).reshape(5, d) + 1
    out = O.combine(y, P.dest_row, w)
    assert np.all(out[5:] == 0) and np.array_equal(out[:5], y)
    sh = np.full((T, d), 7.0)
    out2 = O.combine(y, P.dest_row, w, sh)
    assert np.all(out2[5:] == 7.0)


def test_token_outputs_agree_with_forward():
    r = _rng(18)
    T, d, F, E, k = 30, 8, 6, 4, 2
    x = r.standard_normal((T, d)).astype(np.float32)
    ew = _rand_experts(r, E, d, F)
    sh = _rand_experts(r, 1, d, F)
    spec = O.LayerSpec(T, d, E, k, F, n_shared=1, capacity_factor=1.0)
    res = O.forward(spec, x, r.standard_normal((d, E)).astype(np.float32), ew, sh)
    toks = [0, 3, 29, 17]
    got = O.token_outputs(toks, x, res.perm.dest_row, res.routing.idx, res.routing.w, ew, sh)
    np.testing.assert_allclose(got, res.out[toks], rtol=1e-12, atol=1e-12)


# ------------------------------------------------ load-balancing statistics
def test_router_probs_uniform_logits_give_uniform():
    """Equal logits give 1/E for every expert, in every scoring mode (closed form)."""
    z = np.zeros((3, 6), np.float32)
    for rc in (O.RouteConfig(6, 2), O.RouteConfig(6, 2, tau=0.5),
               O.RouteConfig(6, 2, score=O.SCORE_SIGMOID, bias_mode=O.BIAS_SELECT_ONLY)):
        b = np.linspace(-1, 1, 6).astype(np.float32) if rc.bias_mode else None
        p = O.router_probs(z, rc, b)
        np.testing.assert_allclose(p, 1.0 / 6, rtol=0, atol=1e-15)


def test_router_probs_are_the_unrenormalised_gate_weights():
    """The page's no-renormalisation weights are the top-k entries of the softmax
    over all E, so router_probs at the chosen experts must equal them (Gumbel
    noise and temperature included, as in the perturbed-softmax workload)."""
    r = _rng(11)
    z = r.standard_normal((20, 16)).astype(np.float32)
    u = ((r.integers(0, 1 << 23, (20, 16)) + 0.5) * 2.0 ** -23).astype(np.float32)
    rc = O.RouteConfig(16, 2, renormalize=0, tau=0.5)
    p = O.router_probs(z, rc, None, u)
    ro = O.route_from_logits(z, rc, None, u)
    np.testing.assert_allclose(np.take_along_axis(p, ro.idx.astype(np.int64), 1), ro.w, rtol=2e-7)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-14)


def test_router_probs_ignore_selection_only_bias_and_follow_logit_bias():
    """A selection-only bias steers the top-k but is not part of the probabilities;
    a logit bias of +log(3) on one expert triples its odds against every other."""
    r = _rng(12)
    z = r.standard_normal((7, 5)).astype(np.float32)
    b = r.standard_normal(5).astype(np.float32)
    for score in (O.SCORE_SOFTMAX, O.SCORE_SIGMOID):
        p0 = O.router_probs(z, O.RouteConfig(5, 2, score=score))
        p1 = O.router_probs(z, O.RouteConfig(5, 2, score=score, bias_mode=O.BIAS_SELECT_ONLY), b)
        np.testing.assert_array_equal(p0, p1)
    bl = np.zeros(5, np.float32)
    bl[2] = np.float32(math.log(3.0))
    z0 = np.zeros((1, 5), np.float32)
    p = O.router_probs(z0, O.RouteConfig(5, 1, bias_mode=O.BIAS_LOGIT), bl)[0]
    np.testing.assert_allclose(p[2] / p[0], 3.0, rtol=1e-6)
    np.testing.assert_allclose(p, [1 / 7, 1 / 7, 3 / 7, 1 / 7, 1 / 7], rtol=1e-6)


def test_router_probs_sigmoid_scores_normalised():
    """Sigmoid scoring: logits log(1), log(3) give sigmoid 1/2 and 3/4, so the
    probabilities are 2/5 and 3/5 (hand-computed)."""
    z = np.array([[0.0, math.log(3.0)]], np.float32)
    p = O.router_probs(z, O.RouteConfig(2, 1, score=O.SCORE_SIGMOID))[0]
    np.testing.assert_allclose(p, [0.4, 0.6], rtol=1e-7)


def test_router_stats_hand_example_and_uniform_closed_form():
    """aux = sum_e mean_t(p) * count: p rows (1, 0) and (1/2, 1/2) average to
    (3/4, 1/4); with counts (3, 1) the sum is 3/4*3 + 1/4*1 = 5/2.  With uniform
    probabilities the term is T k / E whatever the counts."""
    P, aux = O.router_stats(np.array([[1.0, 0.0], [0.5, 0.5]]), np.array([3, 1]))
    np.testing.assert_allclose(P, [0.75, 0.25])
    assert aux == pytest.approx(2.5, rel=1e-15)
    r = _rng(13)
    T, E, k = 50, 8, 2
    counts = np.bincount(r.integers(0, E, T * k), minlength=E)
    _, aux_u = O.router_stats(np.full((T, E), 1.0 / E), counts)
    assert aux_u == pytest.approx(T * k / E, rel=1e-13)


def test_bias_update_hand_examples():
    """counts (3, 1): mean 2, ratios (3/2, 1/2); bias (0.2, -0.1) becomes
    (0.99*0.2 - 0.015, 0.99*(-0.1) - 0.005) = (0.183, -0.104).  Balanced counts
    give ratio 1 (every bias decays and drops by the rate); no traffic leaves
    only the decay."""
    b = O.bias_update(np.array([0.2, -0.1], np.float32), np.array([3, 1]))
    np.testing.assert_allclose(b, [0.183, -0.104], rtol=0, atol=1e-7)
    b2 = O.bias_update(np.array([0.5, 0.0, -0.5], np.float32), np.array([4, 4, 4]), 0.9, 0.1)
    np.testing.assert_allclose(b2, [0.35, -0.1, -0.55], rtol=0, atol=1e-7)
    b3 = O.bias_update(np.array([1.0, -2.0], np.float32), np.array([0, 0]))
    np.testing.assert_allclose(b3, [0.99, -1.98], rtol=0, atol=1e-7)
    assert b.dtype == np.float32


# ------------------------------------------------------ overflow re-routing
def _expert_of_rows(P, idx_shape):
    """Final expert of every pair, from the offsets and dest_row (-1 = dropped)."""
    ex = np.full(idx_shape, -1)
    for t in range(idx_shape[0]):
        for j in range(idx_shape[1]):
            r = P.dest_row[t, j]
            if r >= 0:
                ex[t, j] = int(np.searchsorted(P.offsets, r, side="right") - 1)
    return ex


def test_reroute_without_overflow_is_the_plain_permutation():
    r = _rng(21)
    idx = r.integers(0, 6, (40, 2))
    fb = np.tile(np.arange(6), (40, 1))[:, :3]
    for C in (None, 1000):
        a, b = O.permute_reroute(idx, fb, 6, C), O.permute(idx, 6, C)
        for f in ("counts", "kept", "offsets", "dest_row", "src_token"):
            np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
        assert a.n_dropped == b.n_dropped == 0


def test_reroute_hand_example_fills_next_best_free_expert():
    """Four tokens all pick expert 0 (C = 1), each with fallbacks (1, 2): the first
    is kept, the second goes to 1, the third finds 1 full and goes to 2, the
    fourth finds everything full and is dropped."""
    idx = np.zeros((4, 1), np.int32)
    fb = np.tile([1, 2], (4, 1))
    P = O.permute_reroute(idx, fb, 3, 1)
    np.testing.assert_array_equal(_expert_of_rows(P, idx.shape)[:, 0], [0, 1, 2, -1])
    np.testing.assert_array_equal(P.counts, [4, 0, 0])
    np.testing.assert_array_equal(P.kept, [1, 1, 1])
    assert P.n_dropped == 1


def test_reroute_slots_of_one_token_take_distinct_experts_in_key_order():
    """Token 2's two slots both overflow (C = 2) and share fallbacks (2, 3): the
    first slot takes 2; expert 2 still has room, but it already serves the
    token, so the second slot takes 3."""
    idx = np.array([[0, 1], [0, 1], [0, 1]])
    fb = np.array([[2, 3], [2, 3], [2, 3]])
    P = O.permute_reroute(idx, fb, 4, 2)
    np.testing.assert_array_equal(_expert_of_rows(P, idx.shape), [[0, 1], [0, 1], [2, 3]])


def test_reroute_rows_follow_the_first_pass():
    """Token 2 overflows expert 0 (C = 2) and falls back to expert 1, which kept
    token 3 in the first pass: expert 1's rows are token 3 (first pass) then
    token 2 (re-routed), so offsets (0, 2, 4), dest rows 2 and 3."""
    idx = np.array([[0], [0], [0], [1]])
    fb = np.array([[1], [1], [1], [0]])
    P = O.permute_reroute(idx, fb, 2, 2)
    np.testing.assert_array_equal(_expert_of_rows(P, idx.shape)[:, 0], [0, 0, 1, 1])
    np.testing.assert_array_equal(P.offsets, [0, 2, 4])
    np.testing.assert_array_equal(P.dest_row[:, 0], [0, 1, 3, 2])
    np.testing.assert_array_equal(P.src_token, [0, 1, 3, 2])
    assert P.n_dropped == 0


def test_reroute_priority_goes_to_the_earlier_token():
    """Tokens 1 and 2 both overflow expert 0 (C = 1) and both want expert 1, which
    has room for one: token 1 gets it, token 2 falls through to expert 2."""
    idx = np.array([[0], [0], [0]])
    fb = np.array([[1, 2], [1, 2], [1, 2]])
    P = O.permute_reroute(idx, fb, 3, 1)
    np.testing.assert_array_equal(_expert_of_rows(P, idx.shape)[:, 0], [0, 1, 2])


def _deferred_acceptance(idx, fb, E, C):
    """Independent formulation: every token with overflowed slots proposes down
    its fallback list until it holds as many experts as it has such slots; every
    expert keeps the earliest tokens that fit its spare room and rejects the
    rest; rejected tokens propose further, until nothing is rejected.  With one
    priority order shared by all experts this reaches the same assignment as the
    serial rule; a token's experts go to its overflowed slots in list order."""
    T, k = idx.shape
    counts = np.bincount(np.asarray(idx).ravel(), minlength=E)
    rank = np.zeros((T, k), int)
    seen = np.zeros(E, int)
    for t in range(T):
        for j in range(k):
            rank[t, j] = seen[idx[t, j]]
            seen[idx[t, j]] += 1
    room = C - np.minimum(counts, C)
    slots = [[j for j in range(k) if rank[t, j] >= C] for t in range(T)]
    ptr = [0] * T
    held = [set() for _ in range(T)]
    while True:
        for t in range(T):
            while len(held[t]) < len(slots[t]) and ptr[t] < fb.shape[1]:
                held[t].add(int(fb[t, ptr[t]]))
                ptr[t] += 1
        rejected = False
        for c in range(E):
            holders = [t for t in range(T) if c in held[t]]
            for t in holders[room[c]:]:
                held[t].discard(c)
                rejected = True
        if not rejected:
            break
    out = np.where(rank < C, idx, -1)
    for t in range(T):
        mine = [int(c) for c in fb[t] if int(c) in held[t]]
        for j, c in zip(slots[t], mine):
            out[t, j] = c
    return out


def test_reroute_matches_deferred_acceptance_bruteforce():
    """Random tiny cases: the serial rule and deferred acceptance agree."""
    r = _rng(22)
    for trial in range(300):
        E = int(r.integers(2, 7))
        k = int(r.integers(1, min(3, E) + 1))
        D = int(r.integers(1, E - k + 1)) if E > k else 0
        T = int(r.integers(1, 10))
        keys = r.standard_normal((T, E)).astype(np.float32)
        keys[:, 0] += 2.0  # a hot expert, so overflow happens
        idx, _, _ = O.topk_by_keys(keys, k)
        fb = O.fallback_candidates(keys, k, D) if D else np.zeros((T, 0), np.int32)
        C = int(r.integers(1, 4))
        P = O.permute_reroute(idx, fb, E, C)
        np.testing.assert_array_equal(_expert_of_rows(P, idx.shape), _deferred_acceptance(idx, fb, E, C),
                                      err_msg=f"trial {trial}")


def test_reroute_invariants_on_skewed_traffic():
    """Zipf-like traffic: every expert holds at most C rows, a token's experts are
    distinct, rows and tokens agree, and a pair left dropped found every one of its
    fallbacks full or already serving its token."""
    r = _rng(23)
    T, E, k, D, C = 300, 16, 2, 4, 30
    keys = (r.standard_normal((T, E)) - 0.6 * np.arange(E)).astype(np.float32)
    idx, _, _ = O.topk_by_keys(keys, k)
    fb = O.fallback_candidates(keys, k, D)
    P = O.permute_reroute(idx, fb, E, C)
    assert P.kept.max() <= C and P.n_dropped > 0 and P.n_dropped < O.permute(idx, E, C).n_dropped
    ex = _expert_of_rows(P, idx.shape)
    full = P.kept >= C
    for t in range(T):
        mine = [e for e in ex[t] if e >= 0]
        assert len(mine) == len(set(mine))
        for j in range(k):
            if ex[t, j] < 0:
                assert all(full[c] or c in mine for c in fb[t])
    n = int(P.offsets[-1])
    for t in range(T):
        for j in range(k):
            if P.dest_row[t, j] >= 0:
                assert P.src_token[P.dest_row[t, j]] == t
    assert (P.src_token[:n] >= 0).all() and (P.src_token[n:] == -1).all()


def test_rerouted_layer_serves_each_slot_by_its_fallback_expert():
    """A whole layer with re-routing: every kept slot's output row is its serving
    expert's FFN of the token (token_outputs, one token at a time, with the
    serving experts), re-routing keeps more pairs than plain dropping, and a
    dropped slot contributes nothing."""
    r = _rng(24)
    T, d, F, E, k = 40, 8, 6, 6, 2
    x = r.standard_normal((T, d)).astype(np.float32)
    wr = r.standard_normal((d, E)).astype(np.float32)
    wr[:, 0] += 2.0  # a hot expert
    ew = _rand_experts(r, E, d, F)
    spec = O.LayerSpec(T, d, E, k, F, capacity_factor=1.0, reroute_depth=3)
    res = O.forward(spec, x, wr, ew)
    plain = O.forward(O.LayerSpec(T, d, E, k, F, capacity_factor=1.0), x, wr, ew)
    assert res.perm.n_dropped < plain.perm.n_dropped
    serving = O.serving_experts(res.perm)
    assert (serving != res.routing.idx).any()  # some slot moved
    toks = list(range(T))
    got = O.token_outputs(toks, x, res.perm.dest_row, serving, res.routing.w, ew)
    np.testing.assert_allclose(got, res.out, rtol=1e-12, atol=1e-12)


# -------------------------------------------------- group-limited routing
def test_group_limit_hand_example():
    """Keys (5, 1, 4, 3), groups {0,1} {2,3}, one group, top-2: group scores are
    (5, 4), so group 0 is kept and the experts are (0, 1) -- not (0, 2) as
    without groups.  Keeping both groups is plain top-k."""
    keys = np.array([[5.0, 1.0, 4.0, 3.0]], np.float32)
    r = O.route_from_logits(keys, O.RouteConfig(4, 2, n_groups=2, topk_groups=1))
    np.testing.assert_array_equal(r.idx, [[0, 1]])
    r2 = O.route_from_logits(keys, O.RouteConfig(4, 2, n_groups=2, topk_groups=2))
    np.testing.assert_array_equal(r2.idx, [[0, 2]])
    assert r.gap_sel[0] == 1.0  # the group decision: 5 against 4


def test_group_limit_bruteforce():
    """Random keys: the chosen experts are the top-k of the union of the M groups
    with the largest maxima (brute force over every M-subset of groups), and the
    token's best expert is always among them."""
    r = _rng(31)
    for trial in range(200):
        G = int(r.choice([2, 4, 8]))
        gs = int(r.choice([2, 3, 4]))
        E = G * gs
        M = int(r.integers(1, G + 1))
        k = int(r.integers(1, M * gs + 1))
        keys = r.standard_normal((1, E)).astype(np.float32)
        got = O.route_from_logits(keys, O.RouteConfig(E, k, n_groups=G, topk_groups=M)).idx[0]
        gmax = keys[0].reshape(G, gs).max(axis=1)
        best = max(itertools.combinations(range(G), M), key=lambda c: sorted(gmax[list(c)], reverse=True))
        allowed = [e for g in best for e in range(g * gs, (g + 1) * gs)]
        want = sorted(allowed, key=lambda e: -keys[0, e])[:k]
        assert list(got) == want, trial
        assert int(np.argmax(keys[0])) in got


def test_group_limit_off_is_plain_routing():
    r = _rng(32)
    z = r.standard_normal((30, 16)).astype(np.float32)
    for G in (0, 1):
        a = O.route_from_logits(z, O.RouteConfig(16, 3, n_groups=G, topk_groups=1))
        b = O.route_from_logits(z, O.RouteConfig(16, 3))
        np.testing.assert_array_equal(a.idx, b.idx)
        np.testing.assert_array_equal(a.w, b.w)
