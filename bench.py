"""Benchmark of the sparse MoE layer on one MI355X.

One step = one moe_forward call (route -> top-k -> capacity-limited permute ->
grouped SwiGLU experts -> weighted combine) over one batch of seeded synthetic
input already resident in HBM.  Prints one JSON line:

  value       tokens per second of the whole layer (T / step time)
  roofline    the dominant kernel's achieved rate from HIP events recorded
              around each launch on its stream, against the MI355X peak for
              its bound; the events are taken over a second run of the same K
              steps right after the timed one (recording them between kernels
              would lengthen the timed steps themselves)
  kernels     the same for every kernel of the step (average duration,
              algorithmic FLOP or bytes per launch, rate, fraction of peak)
  cpu_baseline the CPU oracle on a bounded sample of the same workload

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 20] [--workload mixtral_bf16]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s; grouped-GEMM % MFMA peak; permute/combine % HBM BW"
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
DEFAULT_WORKLOAD = "mixtral_bf16"


SETTLE_MS = 100.0  # untimed load before the timed steps, at least (warm-up + settle steps)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the GPU clocks take a few tens of milliseconds of load to settle
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=0, help="tokens in the oracle sample (0: auto)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 512 MiB device copy first (HBM counter calibration)")
    ap.add_argument("--balance", action="store_true",
                    help="each step also runs the load-balancing statistics and the bias step "
                         "(moe_router_stats, moe_bias_update on a scratch bias)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph holding one step per weight copy "
                         "(the serving mode for decode) instead of stream launches")
    ap.add_argument("--weight-copies", type=int, default=0,
                    help="expert-weight copies the steps rotate through (0: 3 when T <= 1024, else 1), "
                         "so a small step's weights are not served from the 256 MB MALL")
    return ap.parse_args()


def kernel_source_hash() -> str:
    """sha256 over every kernel source; a traffic record taken with other sources
    no longer describes the kernels that run."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_sparse_amd", "csrc")
    files = sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".h")))
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def recorded_traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed rocprofv3 FETCH_SIZE / WRITE_SIZE record
    (profiles/*.md, a line `traffic_record: {json}`), if it was taken on these sources."""
    pdir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None
    want = kernel_source_hash()
    for f in sorted(os.listdir(pdir)):
        if not f.endswith(".md"):
            continue
        with open(os.path.join(pdir, f)) as fh:
            for line in fh:
                if not line.startswith("traffic_record: "):
                    continue
                rec = json.loads(line[len("traffic_record: "):])
                if rec.get("kernel") == kernel and rec.get("workload") == workload \
                        and rec.get("source_sha256") == want:
                    return rec
    return None


def algorithmic_work(sh, kept_rows: int, touched: int):
    """Per-launch algorithmic FLOP and HBM bytes of each kernel (each tensor once)."""
    from mixture_experts_sparse_amd import workloads as W
    a = W.nbytes_of(sh.act_dtype)
    wb = W.nbytes_of(sh.w_dtype)
    hb = 4 if sh.w_dtype == W.DT_F32 else 2
    T, d, E, k, F, N = sh.T, sh.d, sh.E, sh.k, sh.F, kept_rows
    # scales: fp8 one f32 per weight row; INT4 one 32-bit word per 128 weights of a row
    if sh.w_dtype == W.DT_FP8:
        sc_gu, sc_dn = 4 * 2 * F, 4 * d
    elif sh.w_dtype == W.DT_INT4:
        sc_gu, sc_dn = 4 * 2 * F * (d // 128), 4 * d * (F // 128)
    else:
        sc_gu = sc_dn = 0
    ep = 16
    while ep < E:
        ep *= 2
    work = {
        # router GEMM: x once, the split router weights once (algorithmic FLOP: the f32 product)
        "router_mfma": {"flop": 2.0 * T * d * E, "bytes": T * d * a + 3 * ep * d * 2},
        "router_prep": {"bytes": d * E * 4 + 3 * ep * d * 2},
        # top-k: logits in, indices and weights out (the d-slice partials are extra traffic)
        "route_topk": {"bytes": T * E * 4 + T * k * 8},
        "permute_hist": {"bytes": T * k * 4},
        "permute_scan": {"bytes": 0},
        "permute_rank": {"bytes": T * k * 8 + N * 4},
        # read each token row once, write each kept copy once
        "permute_scatter": {"bytes": T * d * a + N * d * a + T * k * 4},
        "gemm_tiles": {"bytes": 0},
        # gate/up: x_perm read, both weight matrices of every touched expert, h written
        "gemm_gate_up": {"flop": 4.0 * N * d * F,
                         "bytes": N * d * a + touched * (2 * F * d * wb + sc_gu) + N * F * hb},
        "gemm_down": {"flop": 2.0 * N * F * d,
                      "bytes": N * F * hb + touched * (d * F * wb + sc_dn) + N * d * 4},
        # kept rows of y (f32) read once, output written once (+ shared rows)
        "combine": {"bytes": N * d * 4 + T * d * (4 if sh.out_dtype == W.DT_F32 else 2)
                    + T * k * 8 + (T * d * 4 if sh.n_shared else 0)},
    }
    # load balancing (--balance): the logits (and Gumbel uniforms) read once
    work["balance_stats"] = {"bytes": T * E * 4 * (2 if sh.gumbel else 1)}
    # one-chunk count/scan/rank: the pair ids in, dest_row and src_token out
    work["permute_count_rank"] = {"bytes": T * k * 8 + N * 4}
    # overflow re-routing: each token's k + D expert ids and its k first-pass rows
    # in, a state word per token out (init); per round the same in, a fallback
    # expert and rank per pair out; the finish kernel sums E counts per block of
    # proposals and writes the offsets; relocation: the pairs again
    D = sh.reroute_depth
    work["permute_reroute_init"] = {"bytes": T * (k + D) * 4 + T * k * 4 + T * 4}
    work["permute_reroute_round"] = {"bytes": T * (k + D) * 4 + T * k * 4 + 2 * T * 4 + 2 * T * k * 4}
    work["permute_reroute_finish"] = {"bytes": -(-T // 256) * E * 4 + 3 * (E + 1) * 4}
    work["permute_relocate"] = {"bytes": T * k * 4 * 4 + N * 4}
    if sh.n_shared:
        work["shared_gate_up"] = {"flop": 4.0 * T * d * F, "bytes": T * d * a + 2 * F * d * wb + sc_gu + T * F * hb}
        work["shared_down"] = {"flop": 2.0 * T * F * d, "bytes": T * F * hb + d * F * wb + sc_dn + T * d * 4}
    return work


def kernel_key(name: str) -> str:
    """Library kernel name -> work key (drops the dtype tags)."""
    for tag in ("_f32", "_bf16", "_fp8", "_int4"):
        name = name.replace(tag, "")
    return name


def host_cpu():
    """Logical CPUs this process may run on, and the CPU model name."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def cpu_baseline(inp, sample: int, one_thread_s: float = 10.0):
    """Time the CPU oracle (as it stands) on the first `sample` tokens with every
    BLAS thread, then on a smaller first slice with one thread (sized to take
    about `one_thread_s` seconds)."""
    import numpy as np  # noqa: F401
    import threadpoolctl

    from oracle import from_inputs as FI
    from oracle import moe_oracle as O

    sh = inp.shape
    cpu = inp.to("cpu")
    ew = FI.expert_weights(cpu)
    shw = FI.shared_weights(cpu)
    wr, b = FI.to_np(cpu.w_router), FI.to_np(cpu.bias)
    x_all = FI.to_np(cpu.x)
    u_all = FI.to_np(cpu.gumbel_u)

    def run(n):
        x = x_all[:n]
        u = None if u_all is None else u_all[:n]
        spec = FI.layer_spec(sh.replace(T=n))
        t0 = time.perf_counter()
        O.forward(spec, x, wr, ew, shw, b, u)
        return time.perf_counter() - t0

    threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1])
    dt = run(sample)
    n1 = int(max(16, min(sample, sample * one_thread_s / max(dt * threads, 1e-9))))
    with threadpoolctl.threadpool_limits(1):
        dt1 = run(n1)
    nproc, model = host_cpu()
    return {"value": sample / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {sample} of {sh.T} tokens of {sh.name} (capacity recomputed for the "
                      f"sample), full layer in float64 numpy; {dt:.2f} s wall with {threads} BLAS "
                      f"threads",
            "nproc": nproc, "cpu_model": model, "wall_s": round(dt, 3),
            "one_thread": {"value": n1 / dt1, "unit": "tokens/s", "tokens": n1, "wall_s": round(dt1, 3)}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer's multi-GPU "
              "sharding is a design note, not a measured path", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from mixture_experts_sparse_amd import load
    from mixture_experts_sparse_amd import workloads as W

    L = load()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    sh = W.WORKLOADS[args.workload]
    print(f"[bench] workload {sh.name}: T={sh.T} d={sh.d} E={sh.E} k={sh.k} F={sh.F}", file=sys.stderr, flush=True)
    if args.calibrate_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    inp = W.make_inputs(sh, device=dev)
    cfg = L.make_config(sh)
    copies = args.weight_copies or (3 if sh.T <= 1024 else 1)
    weight_sets = [L.expert_weights(inp)]
    keep = []
    for _ in range(copies - 1):
        c = inp.clone_weights()
        keep.append(c)
        weight_sets.append(L.expert_weights(c))
    ws = L.alloc_workspace(cfg, dev)
    out = torch.empty((sh.T, sh.d), dtype=torch.float32, device=dev)
    stats = torch.empty(2 * sh.E + 1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    print("[bench] inputs ready", file=sys.stderr, flush=True)

    routing = None
    if args.balance:
        routing = {"logits": torch.empty((sh.T, sh.E), dtype=torch.float32, device=dev)}
        prob_mean = torch.empty(sh.E, dtype=torch.float32, device=dev)
        aux = torch.empty(1, dtype=torch.float32, device=dev)
        scratch_bias = torch.zeros(sh.E, dtype=torch.float32, device=dev)
        counts = stats[: sh.E]

    def step(i):
        L.moe_forward(cfg, inp.x, inp.w_router, inp.bias, inp.gumbel_u, weight_sets[i % copies], out,
                      stats, ws, routing=routing)
        if args.balance:
            L.moe_router_stats(cfg, routing["logits"], inp.bias, inp.gumbel_u, counts, prob_mean, aux, ws)
            L.moe_bias_update(cfg, counts, scratch_bias)

    w0 = torch.cuda.Event(enable_timing=True)
    w1 = torch.cuda.Event(enable_timing=True)
    w0.record()
    for i in range(args.warmup):
        step(i)
    w1.record()
    torch.cuda.synchronize()
    # the clocks need about 100 ms of load to settle: when the W warm-up steps
    # are shorter than that (decode-sized steps), more untimed steps follow
    warm_ms = w0.elapsed_time(w1) if args.warmup else 0.0
    per_ms = warm_ms / args.warmup if args.warmup else 0.0
    settle = 0
    if warm_ms < SETTLE_MS:
        if per_ms <= 0.0:  # no warm-up steps: time one
            w0.record()
            step(0)
            w1.record()
            torch.cuda.synchronize()
            per_ms = max(w0.elapsed_time(w1), 1e-3)
            warm_ms, settle = per_ms, 1
        n = min(20000, int((SETTLE_MS - warm_ms) / per_ms) + 1)
        for i in range(n):
            step(i)
        torch.cuda.synchronize()
        settle += n
    if args.graph:
        # one graph holds one step per weight copy (the library makes no
        # allocation, copy, fill or synchronisation, so a step captures as is)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(copies):
                step(i)
        for _ in range(max(1, args.warmup // copies)):
            graph.replay()
        torch.cuda.synchronize()
        n_calls, per_call = max(1, args.steps // copies), copies

        def run_one(i):
            graph.replay()
    else:
        n_calls, per_call = args.steps, 1

        def run_one(i):
            step(args.warmup + i)
    timed_steps = n_calls * per_call
    # timed region: K steps with an event only at each end (an event between
    # steps lengthens a decode-sized step by a few microseconds)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(n_calls):
        run_one(i)
    t_end.record()
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    # step-time spread: the same steps again, one event after each
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(n_calls + 1)]
    marks[0].record()
    for i in range(n_calls):
        run_one(i)
        marks[i + 1].record()
    torch.cuda.synchronize()
    # per-kernel durations: the same K steps again, with the library's event pair
    # around every launch on its stream (events between kernels lengthen a
    # decode-sized step by up to 75 %, so they stay out of the timed region)
    L.moe_profile_read()  # discard anything recorded before
    L.moe_profile_enable(True)
    for i in range(args.steps):
        step(args.warmup + args.steps + i)
    torch.cuda.synchronize()
    L.moe_profile_enable(False)
    prof = L.moe_profile_read()
    ms_step = ms_total / timed_steps
    step_times = np.array([marks[i].elapsed_time(marks[i + 1]) / per_call for i in range(n_calls)])
    st = stats.cpu().numpy()
    kept = int(st[sh.E:2 * sh.E].sum())
    touched = int((st[sh.E:2 * sh.E] > 0).sum())
    work = algorithmic_work(sh, kept, touched)
    dt_name = {W.DT_BF16: "bf16", W.DT_FP8: "fp8", W.DT_F32: "f32", W.DT_INT4: "int4"}[sh.w_dtype]
    # fp8 and INT4 weights are decoded to bf16 and multiplied on the bf16 MFMA
    mfma_peak = PEAK_TFLOPS["bf16" if sh.w_dtype in (W.DT_FP8, W.DT_INT4) else dt_name]

    kernels = {}
    for name, (launches, total_ms) in prof.items():
        per_step = launches / args.steps
        avg_us = 1000.0 * total_ms / launches
        wk = work.get(kernel_key(name), {})
        flop = wk.get("flop", 0.0)
        byts = wk.get("bytes", 0)
        ent = {"launches_per_step": per_step, "avg_us": round(avg_us, 2)}
        if flop:
            tf = flop / (avg_us * 1e-6) / 1e12
            ent.update({"tflops": round(tf, 1), "mfma_frac": round(tf / mfma_peak, 4)})
        if byts:
            gbs = byts / (avg_us * 1e-6) / 1e9
            ent.update({"gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)})
        kernels[name] = ent

    # dominant kernel: the largest share of the step time
    dom = max(prof.items(), key=lambda kv: kv[1][1])[0]
    dk = kernels[dom]
    rec = recorded_traffic(dom, sh.name)
    traffic = None if rec is None else rec["bytes_per_launch"]
    # the bound is the roof the kernel's own work meets first: its FLOP at the
    # MFMA peak against its bytes at the HBM peak (decode-sized GEMMs stream
    # weights and are HBM-bound; the large-batch ones are MFMA-bound)
    wk = work.get(kernel_key(dom), {})
    t_mfma = wk.get("flop", 0.0) / (mfma_peak * 1e12)
    t_hbm = wk.get("bytes", 0) / (PEAK_HBM_GBS * 1e9)
    if "tflops" in dk and t_mfma >= t_hbm:
        roof = {"kernel": dom, "bound": "mfma", "achieved": dk["tflops"], "peak": mfma_peak,
                "unit": "TFLOP/s", "frac": dk["mfma_frac"], "traffic": traffic}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": dk.get("gbs"), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": dk.get("hbm_frac"), "traffic": traffic}
    if rec is not None:
        roof["traffic_unit"] = "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
        roof["traffic_algorithmic"] = work.get(kernel_key(dom), {}).get("bytes")

    res = {
        "metric": METRIC,
        "value": round(sh.T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": timed_steps,
        "warmup": args.warmup,
        "settle_steps": settle,
        "ms_per_step": round(ms_step, 4),
        "step_ms": {"p10": round(float(np.percentile(step_times, 10)), 4),
                    "median": round(float(np.median(step_times)), 4),
                    "p90": round(float(np.percentile(step_times, 90)), 4)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt_name,
        "data": "synthetic",
        "config": {"workload": sh.name, "T": sh.T, "d": sh.d, "E": sh.E, "top_k": sh.k, "F": sh.F,
                   "n_shared": sh.n_shared, "weights": dt_name, "router": "f32",
                   "capacity_factor": sh.capacity_factor or None, "kept_rows": kept,
                   "touched_experts": touched, "dropped": int(st[2 * sh.E]),
                   "weight_copies": copies, "balance": bool(args.balance),
                   "launch": "hip_graph" if args.graph else "stream"},
        "roofline": roof,
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        sample = args.cpu_sample or min(sh.T, 4096)
        print(f"[bench] cpu oracle on {sample} tokens", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(inp, sample)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
