"""Concurrent callers: host threads that each own a stream and a workspace may
call moe_forward at the same time (the library keeps its error text and
launch-profiling records per thread and its per-device set-up in atomics).
Every result must equal the serial result bit for bit."""
import threading

import pytest
import torch

from mixture_experts_sparse_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

WK = W.WORKLOADS
SHAPES = [
    W.shrink(WK["mixtral_bf16"], T=1000, d=512, F=1024),
    W.shrink(WK["skewed_fp8"], T=700, d=256, F=256).replace(reroute_depth=4),
    WK["skewed_int4_decode"],
]
CALLS = 12


class Caller:
    def __init__(self, lib, sh, dev):
        self.lib, self.sh = lib, sh
        self.inp = W.make_inputs(sh, device=dev)
        self.cfg = lib.make_config(sh)
        self.weights = lib.expert_weights(self.inp)
        self.ws = lib.alloc_workspace(self.cfg, dev)
        self.outs = [torch.empty((sh.T, sh.d), dtype=torch.float32, device=dev) for _ in range(CALLS)]
        self.stats = [torch.empty(2 * sh.E + 1, dtype=torch.int32, device=dev) for _ in range(CALLS)]
        self.stream = torch.cuda.Stream()  # default priority
        self.error = None

    def call(self, i, stream=None):
        inp = self.inp
        self.lib.moe_forward(self.cfg, inp.x, inp.w_router, inp.bias, inp.gumbel_u, self.weights,
                             self.outs[i], self.stats[i], self.ws, stream=stream)

    def run(self, start):
        try:
            start.wait()
            for i in range(CALLS):
                self.call(i, self.stream)
            self.stream.synchronize()
        except Exception as e:  # reported by the main thread
            self.error = e


def test_threads_on_own_streams_match_serial():
    dev = torch.device("cuda:0")
    lib = G.L()
    G.banner("threads: " + ", ".join(f"{s.name} T={s.T} E={s.E}" for s in SHAPES))
    callers = [Caller(lib, sh, dev) for sh in SHAPES]
    refs = []
    for c in callers:  # serial reference on the current stream
        c.call(0)
        torch.cuda.synchronize()
        refs.append((c.outs[0].clone(), c.stats[0].clone()))
        for o in c.outs:
            o.fill_(float("nan"))
    torch.cuda.synchronize()

    start = threading.Barrier(len(callers))
    threads = [threading.Thread(target=c.run, args=(start,)) for c in callers]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=100)
        assert not t.is_alive(), "a caller thread did not finish"
    torch.cuda.synchronize()
    for c, (ref, ref_stats) in zip(callers, refs):
        assert c.error is None, f"{c.sh.name}: {c.error}"
        for i in range(CALLS):
            assert torch.equal(c.outs[i], ref), f"{c.sh.name}: call {i} differs from the serial result"
            assert torch.equal(c.stats[i], ref_stats), f"{c.sh.name}: call {i} stats differ"
