"""Adapters from the seeded workload inputs (torch tensors) to oracle arguments.

Test infrastructure only, like the rest of ``oracle/``.  Conversions are exact:
bf16 -> float32 widening, fp8 codes passed as raw uint8 with their scales.
"""
from __future__ import annotations

import numpy as np
import torch

from . import moe_oracle as O


def to_np(t):
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def scales_np(t):
    """Weight scales: float32 row scales (fp8) as they are; INT4 group words,
    held in int32 tensors, reinterpreted as the uint32 words they are."""
    a = to_np(t)
    return a.view(np.uint32) if a is not None and a.dtype == np.int32 else a


def layer_spec(shape) -> O.LayerSpec:
    """The layer as the C ABI receives it: tau and the capacity factor are float32 there."""
    return O.LayerSpec(shape.T, shape.d, shape.E, shape.k, shape.F, shape.n_shared,
                       shape.score, shape.renormalize, float(np.float32(shape.tau)),
                       shape.bias_mode, float(np.float32(shape.capacity_factor)),
                       shape.reroute_depth, shape.n_groups, shape.topk_groups)


def expert_weights(inp, experts=None) -> O.ExpertWeights:
    """Host copies of the routed experts (all, or only ``experts`` -- others left zero-sized)."""
    if experts is None:
        return O.ExpertWeights(to_np(inp.w_gate), to_np(inp.w_up), to_np(inp.w_down),
                               scales_np(inp.s_gate), scales_np(inp.s_up), scales_np(inp.s_down))
    return _LazyExperts(inp)


class _LazyExperts(O.ExpertWeights):
    """Copies one expert's matrices to the host only when the oracle asks for it."""

    def __init__(self, inp):
        self._inp = inp
        self.w_down = np.empty((0, inp.w_down.shape[1], 0))

    def expert(self, e: int):
        i = self._inp
        sg = None if i.s_gate is None else scales_np(i.s_gate[e])
        su = None if i.s_up is None else scales_np(i.s_up[e])
        sd = None if i.s_down is None else scales_np(i.s_down[e])
        return (O.dequant(to_np(i.w_gate[e]), sg), O.dequant(to_np(i.w_up[e]), su),
                O.dequant(to_np(i.w_down[e]), sd))


def shared_weights(inp):
    if inp.sh_gate is None:
        return None
    return O.ExpertWeights(to_np(inp.sh_gate), to_np(inp.sh_up), to_np(inp.sh_down),
                           scales_np(inp.sh_s_gate), scales_np(inp.sh_s_up), scales_np(inp.sh_s_down))


def forward(inp) -> O.LayerResult:
    """Whole layer on the oracle for (small) workload inputs."""
    return O.forward(layer_spec(inp.shape), to_np(inp.x), to_np(inp.w_router),
                     expert_weights(inp), shared_weights(inp), to_np(inp.bias),
                     to_np(inp.gumbel_u))
