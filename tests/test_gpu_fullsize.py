"""Parity at the full workload sizes, in the launch configuration bench.py times
(one moe_forward call).  Routing and permutation are checked on every token;
the layer output on a seeded sample of tokens the oracle computes one by one."""
import numpy as np
import pytest
import torch

from mixture_experts_sparse_amd import workloads as W
from oracle import from_inputs as FI
from oracle import moe_oracle as O
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

N_SAMPLE = 8


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_fullsize_forward(name):
    assert torch.cuda.is_available()
    sh = W.WORKLOADS[name]
    G.banner(f"full {name} T={sh.T} d={sh.d} E={sh.E} k={sh.k} F={sh.F}")
    inp = W.make_inputs(sh, device="cuda")
    f = G.run_forward(inp)
    rep = {}
    G.check_routing(inp, f, rep)
    P = G.check_permutation(sh, f, rep)
    print({k: v for k, v in rep.items()}, flush=True)
    rng = np.random.default_rng(7)
    # sample tokens that keep at least one assignment (plus one fully dropped, if any)
    kept_any = np.where((f["dest_row"] >= 0).any(1))[0]
    toks = list(rng.choice(kept_any, size=min(N_SAMPLE, len(kept_any)), replace=False))
    dropped_all = np.where((f["dest_row"] < 0).all(1))[0]
    if len(dropped_all):
        toks.append(int(dropped_all[0]))
    toks = np.array(sorted(toks))
    shared = FI.shared_weights(inp)
    ora = O.token_outputs(toks, G.to_np(inp.x), f["dest_row"], O.serving_experts(P), f["topk_w"],
                          FI.expert_weights(inp, experts="lazy"), shared)
    rep["out_err_sampled"] = G.out_err(f["out"][toks], ora)
    rep["tokens"] = toks.tolist()
    print(rep, flush=True)
    assert rep["out_err_sampled"] <= G.TOL_OUT[sh.w_dtype], rep
    if len(dropped_all) and shared is None:
        assert np.all(f["out"][dropped_all] == 0.0)
    del inp
    torch.cuda.empty_cache()
