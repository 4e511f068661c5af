"""Helpers for the GPU parity tests: run the HIP path through the C-ABI binding
and compare with the oracle, with the metrics the layer's parity is defined by.

Metrics
  router logits z  : max |z_gpu - z_ora| / max(|z_ora|, RMS(z_ora))       <= 1e-5
  gate weights w   : max |w_gpu - w_ora| / max(|w_ora|, RMS(w_ora))       <= 1e-5
  expert indices, counts, offsets, permutation: bit-exact (tokens whose
    selection gap is below 1e-5 are set aside for the index-set comparison,
    and those whose order gap is below 1e-5 for the order comparison; both
    are counted and reported)
  layer output     : max |out_gpu - out_ora| / RMS(out_ora over the served tokens)
                     <= 2e-2 (bf16 and INT4 weights), 6e-2 (fp8 weights), 1e-4 (fp32)
    The RMS is taken over the rows the oracle gives a nonzero output (tokens
    that keep at least one expert, or every token with a shared expert): the
    all-zero rows of fully dropped tokens would otherwise shrink the base and
    inflate the metric.  The maximum runs over every element, zero rows included.
    INT4 takes the bf16 bound: its products are exact (bf16 activations times
    the bf16 numbers 128 + q, f32 sums, the group scale applied once per step),
    so its error, like the bf16 path's, comes from rounding h to bf16.
"""
from __future__ import annotations

import numpy as np
import torch

from mixture_experts_sparse_amd import workloads as W
from oracle import from_inputs as FI
from oracle import moe_oracle as O

NEAR_TIE = 1e-5
TOL_Z = 1e-5
TOL_W = 1e-5
TOL_OUT = {W.DT_BF16: 2e-2, W.DT_FP8: 6e-2, W.DT_INT4: 2e-2, W.DT_F32: 1e-4}


def L():
    from mixture_experts_sparse_amd import load
    return load()


def banner(msg: str):
    print(f"\n[gpu-case] {msg}", flush=True)


def rel_err_scaled(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref ** 2)))
    denom = np.maximum(np.abs(ref), rms)
    denom = np.where(denom > 0, denom, 1.0)
    return float(np.max(np.abs(got - ref) / denom))


def served_rms(ref) -> float:
    """RMS of the reference over its rows that are not all zero (all rows if none is)."""
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    if ref.ndim == 2:
        served = np.any(ref != 0.0, axis=1)
        if served.any():
            ref = ref[served]
    return float(np.sqrt(np.mean(ref ** 2)))


def out_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rms = served_rms(ref)
    return float(np.max(np.abs(got - ref))) / (rms if rms > 0 else 1.0)


def oracle_out_on_routing(inp: W.MoEInputs, g: dict, P) -> np.ndarray:
    """The oracle's layer output (float64, every element) for the routing the
    GPU took: its permutation P (checked bit-exact against the GPU's before
    this is called) and its gate weights.  Experts are copied to the host one
    at a time; products are float64 BLAS."""
    x = to_np(inp.x)
    n = int(P.offsets[-1])
    y = O.expert_outputs(x[P.src_token[:n]].astype(np.float64), P.offsets, FI.expert_weights(inp, experts="lazy"))
    y_sh = None
    shared = FI.shared_weights(inp)
    if shared is not None:
        wg, wu, wd = shared.expert(0)
        y_sh = O.swiglu_ffn(x.astype(np.float64), wg, wu, wd)
    return O.combine(y, P.dest_row, g["topk_w"], y_sh)


def to_np(t):
    return FI.to_np(t)


def run_forward(inp: W.MoEInputs, out_dtype=W.DT_F32, ws=None):
    """moe_forward on the GPU; returns host copies of the output, stats and routing."""
    lib = L()
    sh = inp.shape
    cfg = lib.make_config(sh, out_dtype)
    dev = inp.x.device
    T, E, k, d = sh.T, sh.E, sh.k, sh.d
    out = torch.empty((T, d), dtype=torch.float32 if out_dtype == W.DT_F32 else torch.bfloat16, device=dev)
    stats = torch.empty(2 * E + 1, dtype=torch.int32, device=dev)
    routing = {"logits": torch.empty((T, E), dtype=torch.float32, device=dev),
               "topk_idx": torch.empty((T, k + sh.reroute_depth), dtype=torch.int32, device=dev),
               "topk_w": torch.empty((T, k), dtype=torch.float32, device=dev),
               "dest_row": torch.empty((T, k), dtype=torch.int32, device=dev)}
    if ws is None:
        ws = lib.alloc_workspace(cfg, dev)
    lib.moe_forward(cfg, inp.x, inp.w_router, inp.bias, inp.gumbel_u, lib.expert_weights(inp), out,
                    stats, ws, routing=routing)
    torch.cuda.synchronize()
    res = {k_: to_np(v) for k_, v in routing.items()}
    res["out"] = to_np(out)
    res["out_t"] = out
    st = to_np(stats)
    res["counts"], res["kept"], res["n_dropped"] = st[:E], st[E:2 * E], int(st[2 * E])
    return res


def run_stages(inp: W.MoEInputs, out_dtype=W.DT_F32):
    """The four stage entry points called one after the other on the GPU."""
    lib = L()
    sh = inp.shape
    cfg = lib.make_config(sh, out_dtype)
    dev = inp.x.device
    T, E, k, d = sh.T, sh.E, sh.k, sh.d
    R = lib.permuted_rows(cfg)
    ws = lib.alloc_workspace(cfg, dev)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k + sh.reroute_depth), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    lib.moe_route(cfg, inp.x, inp.w_router, inp.bias, inp.gumbel_u, logits, idx, w, ws)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    dest = torch.empty((T, k), dtype=torch.int32, device=dev)
    src = torch.empty(max(R, 1), dtype=torch.int32, device=dev)
    nd = torch.empty(1, dtype=torch.int32, device=dev)
    x_perm = torch.empty((max(R, 1), d), dtype=inp.x.dtype, device=dev)
    lib.moe_permute(cfg, inp.x, idx, counts, offsets, dest, src, nd, x_perm, ws)
    y_perm = torch.empty((max(R, 1), d), dtype=torch.float32, device=dev)
    y_sh = torch.empty((T, d), dtype=torch.float32, device=dev) if sh.n_shared else None
    lib.moe_expert_ffn(cfg, inp.x, x_perm, offsets, lib.expert_weights(inp), y_perm, y_sh, ws)
    out = torch.empty((T, d), dtype=torch.float32 if out_dtype == W.DT_F32 else torch.bfloat16, device=dev)
    lib.moe_combine(cfg, y_perm, y_sh, dest, w, out)
    torch.cuda.synchronize()
    n = int(offsets[-1].item())
    return {"logits": to_np(logits), "topk_idx": to_np(idx), "topk_w": to_np(w), "counts": to_np(counts),
            "offsets": to_np(offsets), "dest_row": to_np(dest), "src_token": to_np(src)[:R],
            "n_dropped": int(nd.item()), "x_perm": to_np(x_perm[:n]), "y_perm": to_np(y_perm[:n]),
            "y_shared": None if y_sh is None else to_np(y_sh), "out": to_np(out), "rows": R}


def oracle_capacity(sh: W.MoEShape):
    # the ABI takes the factor as a float32; the oracle gets that same value
    return O.capacity(sh.T, sh.k, sh.E, float(np.float32(sh.capacity_factor)))


def check_routing(inp: W.MoEInputs, g: dict, report: dict):
    """z within 1e-5; indices bit-exact on the GPU's own z (near-ties set aside); weights within 1e-5."""
    sh = inp.shape
    spec = FI.layer_spec(sh)
    z_ora = O.router_logits(to_np(inp.x), to_np(inp.w_router))
    report["z_err"] = rel_err_scaled(g["logits"], z_ora)
    assert report["z_err"] <= TOL_Z, report
    D = sh.reroute_depth
    r = O.route_from_logits(g["logits"], spec.route, to_np(inp.bias), to_np(inp.gumbel_u), D)
    sel_tie = r.gap_sel < NEAR_TIE
    ord_tie = r.gap_ord < NEAR_TIE
    report["near_tie_sel"] = int(sel_tie.sum())
    report["near_tie_ord"] = int(ord_tie.sum())
    ok = ~sel_tie
    g_idx = g["topk_idx"][:, : sh.k]
    if D:
        # fallback experts, in order, away from near-ties among the first k + D + 1 keys
        keys = r.keys
        if spec.route.n_groups > 1:
            keys, _ = O.group_limited_keys(keys, spec.route.n_groups, spec.route.topk_groups)
        srt = -np.sort(-keys.astype(np.float64), axis=1)[:, : min(sh.k + D + 1, sh.E)]
        fb_tie = np.min(srt[:, :-1] - srt[:, 1:], axis=1) < NEAR_TIE
        report["near_tie_fallback"] = int(fb_tie.sum())
        assert np.array_equal(g["topk_idx"][~fb_tie, sh.k:], r.fallback[~fb_tie]), "fallback experts differ"
    gs = np.sort(g_idx, axis=1)
    os_ = np.sort(r.idx, axis=1)
    assert np.array_equal(gs[ok], os_[ok]), "expert sets differ away from near-ties"
    ok2 = ok & ~ord_tie
    assert np.array_equal(g_idx[ok2], r.idx[ok2]), "expert order differs away from near-ties"
    if ok2.any():
        report["w_err"] = rel_err_scaled(g["topk_w"][ok2], r.w[ok2])
        assert report["w_err"] <= TOL_W, report
    # the oracle's own routing (from its own z) agrees away from near-ties too
    r_own = O.route_from_logits(z_ora, spec.route, to_np(inp.bias), to_np(inp.gumbel_u))
    clear = (r_own.gap_sel > 10 * NEAR_TIE) & ~sel_tie
    report["own_route_flips"] = int((np.sort(r_own.idx, 1) != gs).any(1).sum())
    assert np.array_equal(np.sort(r_own.idx, 1)[clear], gs[clear])
    return r


def check_permutation(sh: W.MoEShape, g: dict, report: dict):
    """The oracle's permutation of the GPU's indices (and, with re-routing, the
    GPU's fallback experts) equals the GPU's, bit for bit."""
    if sh.reroute_depth:
        P = O.permute_reroute(g["topk_idx"][:, : sh.k], g["topk_idx"][:, sh.k:], sh.E, oracle_capacity(sh))
    else:
        P = O.permute(g["topk_idx"], sh.E, oracle_capacity(sh))
    assert np.array_equal(g["counts"], P.counts)
    assert np.array_equal(g["dest_row"], P.dest_row)
    assert g["n_dropped"] == P.n_dropped
    if "kept" in g:
        assert np.array_equal(g["kept"], P.kept)
    if "offsets" in g:
        assert np.array_equal(g["offsets"], P.offsets)
    if "src_token" in g:
        assert np.array_equal(g["src_token"], P.src_token[:len(g["src_token"])])
    report["n_dropped"] = P.n_dropped
    report["kept"] = int(P.kept.sum())
    return P
