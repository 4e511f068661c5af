"""Parity at the full workload sizes, in the launch configuration bench.py times
(one moe_forward call).  Routing and permutation are checked on every token;
the layer output on every element, against the oracle run (float64 BLAS, one
expert at a time) on the routing the GPU took."""
import time

import numpy as np
import pytest
import torch

from mixture_experts_sparse_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


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
    t0 = time.perf_counter()
    ora = G.oracle_out_on_routing(inp, f, P)
    rep["oracle_s"] = round(time.perf_counter() - t0, 1)
    rep["out_err"] = G.out_err(f["out"], ora)
    rep["elements"] = int(ora.size)
    dropped_all = np.where((f["dest_row"] < 0).all(1))[0]
    rep["tokens_all_dropped"] = int(len(dropped_all))
    print(rep, flush=True)
    assert rep["out_err"] <= G.TOL_OUT[sh.w_dtype], rep
    if len(dropped_all) and not sh.n_shared:
        assert np.all(f["out"][dropped_all] == 0.0)
    del inp, ora
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["mixtral_bf16", "fine_shared_bf16", "skewed_fp8_reroute"])
def test_fullsize_forward_is_deterministic(name):
    """Two calls at full size (a fresh workspace for the second) give the same bits:
    no kernel lets the order of arrival decide an order of arithmetic -- the
    stream-K parts are added in part order, the re-routing rounds settle one
    stable assignment, the combine adds its slots in j order."""
    assert torch.cuda.is_available()
    sh = W.WORKLOADS[name]
    G.banner(f"determinism {name} T={sh.T}")
    inp = W.make_inputs(sh, device="cuda")
    a = G.run_forward(inp)
    b = G.run_forward(inp)
    assert np.array_equal(a["out"], b["out"])
    for key in ("topk_idx", "topk_w", "dest_row", "counts", "kept"):
        assert np.array_equal(a[key], b[key]), key
    del inp, a, b
    torch.cuda.empty_cache()
