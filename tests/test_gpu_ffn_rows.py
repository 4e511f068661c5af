"""The expert FFN (moe_expert_ffn) at chosen rows per expert, against the
oracle's expert outputs: counts that put every number of live 16-row groups
into the streaming GEMM's 64- and 32-row tiles (bf16, fp8 and INT4 weights),
and every number of live 16-row groups into both 128-row halves of the
large-tile GEMM's 256-row tiles, next to empty experts; and experts of more
than eight large tiles, whose tiles the large-tile GEMM walks in bands.

y[r] = (silu(x[r] W_gate[e]^T) * (x[r] W_up[e]^T)) W_down[e]^T for the rows r
of expert e (page "GPT-4 has 1.8T parameters but uses 2% per token" (mlqm.cn),
s3.3 SwiGLU; page "MoE sparse activation: principles and engineering
practice" (kapook.pages.dev), s4.2 expert fusion)."""
import numpy as np
import pytest
import torch

from mixture_experts_sparse_amd import workloads as W
from oracle import from_inputs as FI
from oracle import moe_oracle as O
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

# 16 experts each; with k = 1 and no capacity limit the kernel choice follows
# ceil(rows / 16) (the rows per expert the launch plans for):
#   A: 708 rows -> 45 per expert: streaming GEMM, 64-row tiles (bf16 and fp8)
#   B: 454 rows -> 29 per expert: streaming GEMM, 32-row tiles (fp8, INT4)
#   C: 2382 rows -> 149 per expert: large-tile bf16 GEMM (256-row tiles)
COUNTS_A = [1, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64, 65, 97, 0, 130]
COUNTS_B = [1, 15, 16, 17, 31, 32, 33, 0, 5, 20, 40, 50, 63, 64, 65, 2]
COUNTS_C = [1, 31, 32, 33, 127, 128, 129, 255, 256, 257, 300, 0, 513, 64, 96, 160]
# 8 experts, 9867 rows -> 1234 per expert: large tiles; experts of 10, 17 and 9
# m-tiles are walked in 2, 3 and 2 bands (at most 8 m-tiles per band)
COUNTS_D = [2500, 1, 4200, 300, 0, 17, 2049, 800]

CASES = {
    "bf16_tiles64": (W.DT_BF16, COUNTS_A),
    "fp8_tiles64": (W.DT_FP8, COUNTS_A),
    "fp8_tiles32": (W.DT_FP8, COUNTS_B),
    "int4_tiles32": (W.DT_INT4, COUNTS_B),
    "bf16_big": (W.DT_BF16, COUNTS_C),
    "bf16_big_bands": (W.DT_BF16, COUNTS_D),
    # the same experts with F = 4096: the down pass (44 tiles, 64 K steps) is cut
    # into stream-K parts, so parts of banded tiles meet in the partial slots
    "bf16_big_bands_sk": (W.DT_BF16, COUNTS_D),
}
# inner dim per case (256 unless named)
F_OF = {"bf16_big_bands": 512, "bf16_big_bands_sk": 4096}


@pytest.mark.parametrize("name", list(CASES))
def test_expert_ffn_every_live_row_group(name):
    assert torch.cuda.is_available()
    dev = torch.device("cuda")
    w_dtype, counts = CASES[name]
    R = int(sum(counts))
    F = F_OF.get(name, 256)
    sh = W.WORKLOADS["mixtral_bf16"].replace(name=f"rows_{name}", T=R, d=256, E=len(counts), k=1, F=F,
                                             w_dtype=w_dtype)
    G.banner(f"ffn rows {name} R={R} w={w_dtype}")
    inp = W.make_inputs(sh, device=dev)
    lib = G.L()
    cfg = lib.make_config(sh)
    assert lib.permuted_rows(cfg) == R
    offsets_np = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    offsets = torch.from_numpy(offsets_np).to(dev)
    y = torch.full((R, sh.d), float("nan"), dtype=torch.float32, device=dev)
    ws = lib.alloc_workspace(cfg, dev)
    lib.moe_expert_ffn(cfg, None, inp.x, offsets, lib.expert_weights(inp), y, None, ws)
    torch.cuda.synchronize()
    got = G.to_np(y)
    ref = O.expert_outputs(G.to_np(inp.x).astype(np.float64), offsets_np, FI.expert_weights(inp))
    assert np.all(np.isfinite(got)), "a row was not written"
    err = G.out_err(got, ref)
    # per expert too, so a wrong tile names its expert
    worst = max((G.out_err(got[a:b], ref[a:b]), e) for e, (a, b) in
                enumerate(zip(offsets_np[:-1], offsets_np[1:])) if b > a)
    print({"case": name, "rows": R, "y_err": err, "worst_expert": worst}, flush=True)
    tol = G.TOL_OUT[w_dtype]
    assert err <= tol and worst[0] <= tol, (err, worst)
