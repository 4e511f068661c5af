"""moe_forward captured into a HIP graph: the library allocates, copies, fills
and synchronises nothing, so a step captures as is.  Every replay, with eager
calls of the library in between, must equal the eager result bit for bit (the
kernels decide no order by atomics)."""
import pytest
import torch

from mixture_experts_sparse_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

WK = W.WORKLOADS
CASES = {
    "fp8_decode": WK["skewed_fp8_decode"],
    "int4_decode": WK["skewed_int4_decode"],
    "mixtral_small": W.shrink(WK["mixtral_bf16"], T=1000, d=512, F=1024),
    "reroute_small": W.shrink(WK["skewed_fp8"], T=700, d=256, F=256).replace(reroute_depth=4),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(name):
    sh = CASES[name]
    dev = torch.device("cuda:0")
    lib = G.L()
    inp = W.make_inputs(sh, device=dev)
    cfg = lib.make_config(sh)
    weights = lib.expert_weights(inp)
    ws = lib.alloc_workspace(cfg, dev)
    stats = torch.empty(2 * sh.E + 1, dtype=torch.int32, device=dev)
    eager = torch.empty((sh.T, sh.d), dtype=torch.float32, device=dev)
    lib.moe_forward(cfg, inp.x, inp.w_router, inp.bias, inp.gumbel_u, weights, eager, stats, ws)
    torch.cuda.synchronize()
    ref = eager.clone()
    ref_stats = stats.clone()

    out = torch.empty_like(eager)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lib.moe_forward(cfg, inp.x, inp.w_router, inp.bias, inp.gumbel_u, weights, out, stats, ws)
    for rep in range(3):
        out.fill_(float("nan"))
        stats.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs from the eager result"
        assert torch.equal(stats, ref_stats), f"replay {rep}: routing statistics differ"
        # eager work of the library between replays (same workspace, other output)
        lib.moe_forward(cfg, inp.x, inp.w_router, inp.bias, inp.gumbel_u, weights, eager, stats, ws)
        torch.cuda.synchronize()
        assert torch.equal(eager, ref)
