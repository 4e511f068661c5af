"""Seeded synthetic inputs: shapes, determinism, and the routing structure the
workloads are meant to have (checked through the oracle, CPU only)."""
import numpy as np
import torch

from mixture_experts_sparse_amd import workloads as W
from oracle import moe_oracle as O


def test_inputs_are_seeded_and_shaped():
    sh = W.shrink(W.WORKLOADS["fine_shared_bf16"], T=40, d=64, F=32)
    a, b = W.make_inputs(sh), W.make_inputs(sh)
    assert a.x.dtype == torch.bfloat16 and a.x.shape == (40, 64)
    assert a.w_gate.shape == (256, 32, 64) and a.w_down.shape == (256, 64, 32)
    assert a.sh_gate.shape == (1, 32, 64)
    assert torch.equal(a.x, b.x) and torch.equal(a.w_down, b.w_down) and torch.equal(a.bias, b.bias)
    c = W.make_inputs(sh, seed=99)
    assert not torch.equal(a.x, c.x)


def test_fp8_inputs_are_codes_with_row_scales():
    sh = W.shrink(W.WORKLOADS["skewed_fp8"], T=8, d=128, F=64)
    i = W.make_inputs(sh)
    assert i.w_gate.dtype == torch.uint8 and i.s_gate.shape == (128, 64)
    dec = O.dequant(i.w_gate[3].numpy(), i.s_gate[3].numpy())
    # each row reaches +-448 * scale exactly once it is scaled back
    np.testing.assert_allclose(np.abs(dec).max(1), 448.0 * i.s_gate[3].numpy(), rtol=1e-6)
    assert np.abs(dec).max() < 0.2


def test_int4_inputs_are_groups_that_round_trip():
    """INT4 inputs: packed codes [E, rows, cols/2], one word per 128 columns; the
    oracle's decode of them is within half a step (plus the fp16 rounding of the
    scale) of the float32 weights they were made from, and the extreme weights
    of each group land on codes 0 and 15."""
    sh = W.shrink(W.WORKLOADS["skewed_int4_decode"], T=8, d=256, F=384)
    i = W.make_inputs(sh)
    assert i.w_gate.dtype == torch.uint8 and i.w_gate.shape == (128, 384, 128)
    assert i.s_gate.dtype == torch.int32 and i.s_gate.shape == (128, 384, 2)
    assert i.w_down.shape == (128, 256, 192) and i.s_down.shape == (128, 256, 3)
    w32 = W._normal((384, 256), 0.02, W.child_seed(sh.seed, "w_gate", 5), "cpu").double().numpy()
    qp = i.s_gate[5].numpy().view(np.uint32)
    dec = O.dequant(i.w_gate[5].numpy(), qp)
    step = np.repeat((qp & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64), 128, axis=1)
    assert np.all(np.abs(dec - w32) <= 0.51 * step)
    p = i.w_gate[5].numpy()
    codes = np.empty((384, 256), np.int64)
    codes[:, 0::2], codes[:, 1::2] = p & 15, p >> 4
    g = w32.reshape(384, 2, 128)
    cg = codes.reshape(384, 2, 128)
    r, gi = np.meshgrid(np.arange(384), np.arange(2), indexing="ij")
    assert np.all(cg[r, gi, g.argmin(-1)] == 0) and np.all(cg[r, gi, g.argmax(-1)] == 15)


def test_gumbel_uniforms_are_open_interval_float32():
    u = W.gumbel_uniforms(W.WORKLOADS["gumbel_bf16"])
    assert u.dtype == np.float32 and u.shape == (2048, 16)
    assert u.min() > 0 and u.max() < 1
    assert np.all(np.isfinite(O.gumbel_noise(u)))


def test_skewed_workload_hot_expert_near_60_percent():
    """The Zipf(1.2) logit bias puts the hottest expert in ~60 % of top-2 sets."""
    sh = W.WORKLOADS["skewed_fp8"]
    x = W._normal((sh.T, sh.d), 1.0, W.child_seed(sh.seed, "x"), "cpu").to(torch.bfloat16).float().numpy()
    wr = W._normal((sh.d, sh.E), 0.02, W.child_seed(sh.seed, "w_router"), "cpu").numpy()
    z = O.router_logits(x, wr)
    r = O.route_from_logits(z, O.RouteConfig(sh.E, sh.k, bias_mode=O.BIAS_LOGIT), bias=W.zipf_bias(sh))
    cnt = np.bincount(r.idx.ravel(), minlength=sh.E)
    assert 0.55 < cnt.max() / sh.T < 0.65
    P = O.permute(r.idx, sh.E, O.capacity(sh.T, sh.k, sh.E, sh.capacity_factor))
    assert P.kept.max() == 320 and P.n_dropped > 0
