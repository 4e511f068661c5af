"""moe_forward_noalloc (the entry point for callers that cannot allocate):
through the C ABI, two calls in a row on one device -- the second with a
smaller batch, so it runs on the scratch the first call left behind -- each
bit-identical to moe_forward with a workspace of its own; a layer too large for
the scratch is refused before anything is launched."""
import dataclasses

import numpy as np
import pytest
import torch

from mixture_experts_sparse_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

WK = W.WORKLOADS

# (layer, larger batch, smaller batch): the Mixtral-shaped layer (streaming
# GEMMs at 64 rows per expert), the fp8 decode layer under its capacity limit
# (C = 1, then C = 1 with 8 tokens), and a 256-expert sigmoid layer with a
# shared expert and a selection-only bias
PAIRS = {
    "mixtral": (WK["mixtral_bf16"], 256, 64),
    "fp8_decode": (WK["skewed_fp8_decode"], 32, 8),
    "fine_shared": (W.shrink(WK["fine_shared_bf16"], T=96, d=1024, F=512), 96, 40),
}


def _first_tokens(inp: W.MoEInputs, T: int) -> W.MoEInputs:
    """The same layer (weights, router, bias) on the first T tokens."""
    u = None if inp.gumbel_u is None else inp.gumbel_u[:T].contiguous()
    return dataclasses.replace(inp, shape=inp.shape.replace(T=T), x=inp.x[:T].contiguous(), gumbel_u=u)


def _outputs(inp: W.MoEInputs, dev):
    sh = inp.shape
    out = torch.full((sh.T, sh.d), float("nan"), dtype=torch.float32, device=dev)
    stats = torch.full((2 * sh.E + 1,), -7, dtype=torch.int32, device=dev)
    routing = {"logits": torch.empty((sh.T, sh.E), dtype=torch.float32, device=dev),
               "topk_idx": torch.empty((sh.T, sh.k + sh.reroute_depth), dtype=torch.int32, device=dev),
               "topk_w": torch.empty((sh.T, sh.k), dtype=torch.float32, device=dev),
               "dest_row": torch.empty((sh.T, sh.k), dtype=torch.int32, device=dev)}
    return out, stats, routing


def _same(a, b):
    out_a, st_a, r_a = a
    out_b, st_b, r_b = b
    assert torch.equal(out_a, out_b)
    assert torch.equal(st_a, st_b)
    for key in r_a:
        assert torch.equal(r_a[key], r_b[key]), key


@pytest.mark.parametrize("name", list(PAIRS))
def test_noalloc_matches_forward_on_two_calls(name):
    assert torch.cuda.is_available()
    dev = torch.device("cuda")
    lib = G.L()
    layer, t_big, t_small = PAIRS[name]
    G.banner(f"noalloc {name}: T={t_big} then T={t_small} (d={layer.d} E={layer.E} k={layer.k} F={layer.F})")
    full = W.make_inputs(layer.replace(T=t_big), device=dev)
    runs = [_first_tokens(full, t_big), _first_tokens(full, t_small)]
    cfgs = [lib.make_config(r.shape) for r in runs]
    for c in cfgs:
        assert lib.workspace_bytes(c) <= lib.MOE_NOALLOC_SCRATCH_BYTES
    # two allocation-free calls in a row, then the reference calls
    got = []
    for r, c in zip(runs, cfgs):
        o = _outputs(r, dev)
        lib.moe_forward_noalloc(c, r.x, r.w_router, r.bias, r.gumbel_u, lib.expert_weights(r), o[0], o[1],
                                routing=o[2])
        got.append(o)
    torch.cuda.synchronize()
    for r, c, g in zip(runs, cfgs, got):
        ref = _outputs(r, dev)
        ws = lib.alloc_workspace(c, dev)
        lib.moe_forward(c, r.x, r.w_router, r.bias, r.gumbel_u, lib.expert_weights(r), ref[0], ref[1], ws,
                        routing=ref[2])
        torch.cuda.synchronize()
        assert not torch.isnan(g[0]).any()
        _same(g, ref)
    # and the output is the layer's: within the tolerance of the oracle on the GPU's routing
    r, g = runs[1], got[1]
    f = {"topk_idx": G.to_np(g[2]["topk_idx"]), "topk_w": G.to_np(g[2]["topk_w"]),
         "dest_row": G.to_np(g[2]["dest_row"]), "logits": G.to_np(g[2]["logits"])}
    st = G.to_np(g[1])
    E = r.shape.E
    f["counts"], f["kept"], f["n_dropped"] = st[:E], st[E:2 * E], int(st[2 * E])
    rep = {}
    P = G.check_permutation(r.shape, f, rep)
    rep["out_err"] = G.out_err(G.to_np(g[0]), G.oracle_out_on_routing(r, f, P))
    print(rep, flush=True)
    assert rep["out_err"] <= G.TOL_OUT[r.shape.w_dtype], rep


def test_noalloc_refuses_a_layer_larger_than_its_scratch():
    assert torch.cuda.is_available()
    dev = torch.device("cuda")
    lib = G.L()
    sh = WK["mixtral_bf16"].replace(T=1024)
    cfg = lib.make_config(sh)
    assert lib.workspace_bytes(cfg) > lib.MOE_NOALLOC_SCRATCH_BYTES
    inp = W.make_inputs(sh, device=dev)
    out = torch.full((sh.T, sh.d), 3.0, dtype=torch.float32, device=dev)
    with pytest.raises(lib.MoEError) as ei:
        lib.moe_forward_noalloc(cfg, inp.x, inp.w_router, None, None, lib.expert_weights(inp), out, None)
    assert ei.value.status == 2 and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
