"""GPU parity of the load-balancing statistics and the loss-free bias step
(moe_router_stats, moe_bias_update) against the oracle, through the C ABI.

The statistics are checked on the GPU's own router logits (so routing near-ties
cannot make the two sides see different counts); the bias step is checked bit
for bit, and a few balancing steps in a loop are followed against the oracle.
"""
import numpy as np
import pytest
import torch

from mixture_experts_sparse_amd import workloads as W
from oracle import from_inputs as FI
from oracle import moe_oracle as O
from tests import gpu_util as G
from tests.test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu

TOL_P = 1e-6    # f32 rounding of float64 sums taken in another order
TOL_AUX = 1e-6
# every scoring mode: softmax renormalised, perturbed softmax without
# renormalisation, sigmoid with a selection-only bias, Zipf logit bias, odd E,
# E = 256 (four experts per lane), fp32, one token
CASES = ["mixtral_small", "gumbel_small", "fine_shared_small", "skewed_fp8_small", "odd_experts",
         "tiny_fp32", "single_token"]
DECAY, RATE = float(np.float32(0.99)), float(np.float32(0.01))


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda")


def _forward_with_logits(inp, dev):
    lib = G.L()
    sh = inp.shape
    cfg = lib.make_config(sh)
    ws = lib.alloc_workspace(cfg, dev)
    out = torch.empty((sh.T, sh.d), dtype=torch.float32, device=dev)
    stats = torch.empty(2 * sh.E + 1, dtype=torch.int32, device=dev)
    logits = torch.empty((sh.T, sh.E), dtype=torch.float32, device=dev)
    lib.moe_forward(cfg, inp.x, inp.w_router, inp.bias, inp.gumbel_u, lib.expert_weights(inp), out, stats, ws,
                    routing={"logits": logits})
    return cfg, ws, logits, stats


@pytest.mark.parametrize("name", CASES)
def test_router_stats_match_oracle(name, dev):
    sh = SMALL[name]
    G.banner(f"router stats {sh.name} T={sh.T} E={sh.E} k={sh.k}")
    inp = W.make_inputs(sh, device=dev)
    lib = G.L()
    cfg, ws, logits, stats = _forward_with_logits(inp, dev)
    counts = stats[: sh.E].contiguous()
    pm = torch.empty(sh.E, dtype=torch.float32, device=dev)
    aux = torch.empty(1, dtype=torch.float32, device=dev)
    lib.moe_router_stats(cfg, logits, inp.bias, inp.gumbel_u, counts, pm, aux, ws)
    torch.cuda.synchronize()
    spec = FI.layer_spec(sh)
    probs = O.router_probs(G.to_np(logits), spec.route, G.to_np(inp.bias), G.to_np(inp.gumbel_u))
    P, a = O.router_stats(probs, G.to_np(counts))
    np.testing.assert_allclose(G.to_np(pm), P, rtol=TOL_P, atol=1e-12)
    assert float(aux.item()) == pytest.approx(a, rel=TOL_AUX)
    # the counts the statistics used are the routing's own
    assert int(G.to_np(counts).sum()) == sh.T * sh.k


def test_router_stats_empty_batch(dev):
    sh = SMALL["mixtral_small"].replace(T=0)
    lib = G.L()
    cfg = lib.make_config(sh)
    ws = lib.alloc_workspace(cfg, dev)
    counts = torch.zeros(sh.E, dtype=torch.int32, device=dev)
    pm = torch.full((sh.E,), 7.0, dtype=torch.float32, device=dev)
    aux = torch.full((1,), 7.0, dtype=torch.float32, device=dev)
    lib.moe_router_stats(cfg, None, None, None, counts, pm, aux, ws)
    torch.cuda.synchronize()
    assert torch.all(pm == 0) and float(aux.item()) == 0.0


@pytest.mark.parametrize("E", [1, 5, 64, 200, 256])
def test_bias_update_bit_exact(E, dev):
    G.banner(f"bias update E={E}")
    r = np.random.default_rng(E)
    sh = SMALL["mixtral_small"].replace(E=E, k=1)
    lib = G.L()
    cfg = lib.make_config(sh)
    b0 = r.standard_normal(E).astype(np.float32)
    for counts_np in (r.integers(0, 1000, E).astype(np.int32), np.zeros(E, np.int32),
                      np.full(E, 17, np.int32)):
        bias = torch.from_numpy(b0.copy()).to(dev)
        counts = torch.from_numpy(counts_np).to(dev)
        lib.moe_bias_update(cfg, counts, bias, DECAY, RATE)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(G.to_np(bias), O.bias_update(b0, counts_np, DECAY, RATE))


def test_balancing_loop_follows_oracle(dev):
    """Fine-grained routing (sigmoid scores, selection-only bias): forward, update
    the bias from the counts, repeat.  The GPU's counts and biases follow the
    oracle's step by step, and the busiest expert's load falls."""
    sh = SMALL["fine_shared_small"]
    G.banner(f"balancing loop {sh.name}")
    inp = W.make_inputs(sh, device=dev)
    lib = G.L()
    rate = float(np.float32(0.05))  # a faster step than the page's 0.01, so five steps show the effect
    spec = FI.layer_spec(sh)
    bias_o = G.to_np(inp.bias).copy()
    max_load = []
    for step in range(5):
        cfg, ws, logits, stats = _forward_with_logits(inp, dev)
        counts = stats[: sh.E].contiguous()
        torch.cuda.synchronize()
        r = O.route_from_logits(G.to_np(logits), spec.route, bias_o, None)
        assert not (r.gap_sel < G.NEAR_TIE).any(), "a near-tie would make the trajectories diverge"
        counts_o = np.bincount(r.idx.ravel(), minlength=sh.E).astype(np.int32)
        np.testing.assert_array_equal(G.to_np(counts), counts_o)
        max_load.append(int(counts_o.max()))
        lib.moe_bias_update(cfg, counts, inp.bias, DECAY, rate)  # in place: the next step routes with it
        torch.cuda.synchronize()
        bias_o = O.bias_update(bias_o, counts_o, DECAY, rate)
        np.testing.assert_array_equal(G.to_np(inp.bias), bias_o)
    assert max_load[-1] < max_load[0], max_load
