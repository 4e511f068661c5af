"""Workload definitions and seeded synthetic inputs for the sparse MoE layer.

This module only *draws* inputs.  It holds none of the layer's arithmetic:
no routing, no capacity, no FFN, no combine.  Both the HIP path (through the
C-ABI binding) and the CPU oracle consume exactly the tensors produced here.

Shapes and value distributions follow the five workloads the MoE layer is
benchmarked on (tiny fp32 toy, Mixtral-shaped, Gumbel-routed, fine-grained
with a shared expert, skewed fp8 with a capacity limit).  The pages measure on
proprietary traffic; seeded Gaussian hidden states and weights stand in for it.

Random streams: every tensor (and every expert of a weight tensor) gets its
own child seed derived from ``(seed, tensor id, expert)`` with numpy's
``SeedSequence``; values are drawn by torch's generator *on the device the
tensor lives on*.  A seed therefore fixes the values for a given device type
(CPU draws and GPU draws differ, each is reproducible).  Gumbel uniforms and
the Zipf bias permutation are drawn on the host with numpy, so they are the
same everywhere.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch

# ----------------------------------------------------------------------------
# enums mirrored from include/moe.h (kept as plain ints)
SCORE_SOFTMAX, SCORE_SIGMOID = 0, 1
BIAS_NONE, BIAS_LOGIT, BIAS_SELECT_ONLY = 0, 1, 2
DT_F32, DT_BF16, DT_FP8, DT_INT4 = 0, 1, 2, 3

FP8_E4M3FN_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class MoEShape:
    """One MoE-layer workload: problem sizes, routing mode and dtypes."""

    name: str
    T: int                      # tokens
    d: int                      # hidden size
    E: int                      # routed experts
    k: int                      # top-k
    F: int                      # expert inner (intermediate) size
    n_shared: int = 0           # always-on shared experts (0 or 1)
    score: int = SCORE_SOFTMAX
    renormalize: int = 1        # gate weights renormalised over the chosen k
    tau: float = 1.0
    bias_mode: int = BIAS_NONE
    capacity_factor: float = 0.0  # <= 0: no capacity limit
    act_dtype: int = DT_BF16
    w_dtype: int = DT_BF16
    gumbel: bool = False
    bias_kind: str = "none"     # "none" | "normal0.5" | "zipf1.2"
    seed: int = 1234
    out_dtype: int = DT_F32
    reroute_depth: int = 0      # overflow re-routing: fallback experts per token (0 = off)
    n_groups: int = 0           # group-limited routing: expert groups (0 = off)
    topk_groups: int = 0        # groups kept per token

    def replace(self, **kw) -> "MoEShape":
        return dataclasses.replace(self, **kw)

    @property
    def pairs(self) -> int:
        return self.T * self.k


# The five benchmark workloads (index = seed offset).  Sizes are the full ones.
WORKLOADS: Dict[str, MoEShape] = {
    # tiny fp32 toy: softmax -> top-2 renormalised, no capacity limit
    "tiny_fp32": MoEShape("tiny_fp32", T=64, d=128, E=8, k=2, F=256,
                          act_dtype=DT_F32, w_dtype=DT_F32, seed=1234),
    # Mixtral-shaped: bf16 weights/activations, fp32 router and accumulation
    "mixtral_bf16": MoEShape("mixtral_bf16", T=4096, d=4096, E=8, k=2, F=14336,
                             seed=1235),
    # Gumbel-routed, d=12800, 16 experts, tau=0.5, softmax over all E (no renorm)
    "gumbel_bf16": MoEShape("gumbel_bf16", T=2048, d=12800, E=16, k=2, F=5120,
                            tau=0.5, renormalize=0, gumbel=True, seed=1236),
    # fine-grained 256 experts top-8 + 1 shared expert, sigmoid scores,
    # selection-only per-expert bias ~ N(0, 0.5^2)
    "fine_shared_bf16": MoEShape("fine_shared_bf16", T=8192, d=7168, E=256, k=8,
                                 F=2048, n_shared=1, score=SCORE_SIGMOID,
                                 bias_mode=BIAS_SELECT_ONLY, bias_kind="normal0.5",
                                 seed=1237),
    # skewed, capacity-limited, fp8 e4m3fn weights with per-row fp32 scales
    "skewed_fp8": MoEShape("skewed_fp8", T=16384, d=4096, E=128, k=2, F=1536,
                           bias_mode=BIAS_LOGIT, bias_kind="zipf1.2",
                           capacity_factor=1.25, w_dtype=DT_FP8, seed=1238),
    # the fine-grained layer with group-limited routing: 8 groups of 32, 4 kept
    "fine_grouped_bf16": MoEShape("fine_grouped_bf16", T=8192, d=7168, E=256, k=8, F=2048, n_shared=1,
                                  score=SCORE_SIGMOID, bias_mode=BIAS_SELECT_ONLY, bias_kind="normal0.5",
                                  seed=1237, n_groups=8, topk_groups=4),
    # the skewed layer with overflow re-routing to the four next-best experts
    "skewed_fp8_reroute": MoEShape("skewed_fp8_reroute", T=16384, d=4096, E=128, k=2, F=1536,
                                   bias_mode=BIAS_LOGIT, bias_kind="zipf1.2", capacity_factor=1.25,
                                   w_dtype=DT_FP8, seed=1238, reroute_depth=4),
    # the same layer at decode size (weight-streaming bound)
    "skewed_fp8_decode": MoEShape("skewed_fp8_decode", T=32, d=4096, E=128, k=2,
                                  F=1536, bias_mode=BIAS_LOGIT, bias_kind="zipf1.2",
                                  capacity_factor=1.25, w_dtype=DT_FP8, seed=1238),
    # decode size with group-wise INT4 expert weights (128 per group, fp16 scale
    # and 4-bit zero point per group), bf16 activations, fp32 router
    "skewed_int4_decode": MoEShape("skewed_int4_decode", T=32, d=4096, E=128, k=2,
                                   F=1536, bias_mode=BIAS_LOGIT, bias_kind="zipf1.2",
                                   capacity_factor=1.25, w_dtype=DT_INT4, seed=1238),
}

# Zipf exponent of the skewed workload, and the logit-scale lambda that turns
# log-probabilities into a bias (b_e = lambda * ln p_e).  lambda = 0.94 makes
# the hottest expert appear in ~60 % of the tokens' top-2 at d=4096 with the
# N(0,1) x N(0,0.02^2) router (checked by a CPU test through the oracle).
ZIPF_S = 1.2
ZIPF_LAMBDA = 0.94

_TENSOR_IDS = {"x": 1, "w_router": 2, "w_gate": 3, "w_up": 4, "w_down": 5,
               "sh_gate": 6, "sh_up": 7, "sh_down": 8, "bias": 9, "gumbel": 10,
               "zipf_perm": 11}


def child_seed(seed: int, tensor: str, index: int = 0) -> int:
    """Independent 63-bit seed for (seed, tensor, index)."""
    ss = np.random.SeedSequence(seed, spawn_key=(_TENSOR_IDS[tensor], index))
    return int(ss.generate_state(1, dtype=np.uint64)[0]) & ((1 << 63) - 1)


def _normal(shape, std: float, seed: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def quantize_rows_fp8(w: torch.Tensor):
    """Per-output-row e4m3fn quantisation of a float32 [..., rows, cols] tensor.

    scale[row] = max_i |w[row, i]| / 448; code = RNE(w / scale) saturated to
    +-448.  Returns (codes as uint8 tensor, float32 scales).  This is how the
    fp8 workload's *inputs* are made; the layer itself only ever decodes them.
    """
    amax = w.abs().amax(dim=-1, keepdim=True)
    scale = torch.where(amax > 0, amax / FP8_E4M3FN_MAX, torch.ones_like(amax))
    q = (w / scale).clamp_(-FP8_E4M3FN_MAX, FP8_E4M3FN_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale.squeeze(-1).contiguous()


INT4_GROUP = 128


def quantize_groups_int4(w: torch.Tensor):
    """Group-wise asymmetric INT4 quantisation of a float32 [..., rows, cols]
    tensor, 128 consecutive columns per group: scale = (max - min) / 15 (1 when
    the group is constant), zero = clamp(RNE(-min / scale), 0, 15), code =
    clamp(RNE(w / scale) + zero, 0, 15).  Returns (codes packed two per byte, the
    even column in the low nibble, uint8 [..., rows, cols/2]; group parameters
    [..., rows, cols/128], each the 32-bit word fp16 scale bits | zero << 16,
    held in an int32 tensor).  This is how the INT4
    workload's *inputs* are made; the layer itself only ever decodes them."""
    g = w.reshape(*w.shape[:-1], w.shape[-1] // INT4_GROUP, INT4_GROUP)
    lo, hi = g.amin(dim=-1, keepdim=True), g.amax(dim=-1, keepdim=True)
    scale = torch.where(hi > lo, (hi - lo) / 15.0, torch.ones_like(hi))
    zero = torch.round(-lo / scale).clamp_(0, 15)
    q = (torch.round(g / scale) + zero).clamp_(0, 15).to(torch.uint8).reshape(w.shape)
    packed = (q[..., 0::2] | (q[..., 1::2] << 4)).contiguous()
    s16 = scale.squeeze(-1).to(torch.float16).view(torch.int16).to(torch.int64) & 0xFFFF
    qp = (s16 | (zero.squeeze(-1).to(torch.int64) << 16)).to(torch.int32).contiguous()
    return packed, qp


def _store_weight(w32: torch.Tensor, w_dtype: int):
    if w_dtype == DT_F32:
        return w32, None
    if w_dtype == DT_BF16:
        return w32.to(torch.bfloat16), None
    if w_dtype == DT_FP8:
        return quantize_rows_fp8(w32)
    if w_dtype == DT_INT4:
        return quantize_groups_int4(w32)
    raise ValueError(w_dtype)


def _expert_tensor(shape: MoEShape, name: str, n_exp: int, rows: int, cols: int,
                   device, w_dtype: int):
    """[n_exp, rows, cols] weights ~ N(0, 0.02^2), drawn expert by expert."""
    if w_dtype == DT_F32:
        dt = torch.float32
    elif w_dtype == DT_BF16:
        dt = torch.bfloat16
    else:
        dt = torch.uint8
    out = torch.empty((n_exp, rows, cols // 2 if w_dtype == DT_INT4 else cols), dtype=dt, device=device)
    if w_dtype == DT_FP8:
        scales = torch.empty((n_exp, rows), dtype=torch.float32, device=device)
    elif w_dtype == DT_INT4:
        scales = torch.empty((n_exp, rows, cols // INT4_GROUP), dtype=torch.int32, device=device)
    else:
        scales = None
    # experts are drawn one by one (one seed each) into a float32 chunk of at
    # most ~1 GiB, which is scaled and stored in one go: every step is
    # elementwise or reduces within a row, so the result does not depend on
    # the chunking, and far fewer small launches are made than expert by expert
    chunk = max(1, min(n_exp, (1 << 30) // max(1, rows * cols * 4)))
    for e0 in range(0, n_exp, chunk):
        n = min(chunk, n_exp - e0)
        w32 = torch.empty((n, rows, cols), dtype=torch.float32, device=device)
        for i in range(n):
            g = torch.Generator(device=device)
            g.manual_seed(child_seed(shape.seed, name, e0 + i))
            torch.randn((rows, cols), generator=g, out=w32[i])
        w32.mul_(0.02)
        w, s = _store_weight(w32, w_dtype)
        out[e0:e0 + n].copy_(w)
        if scales is not None:
            scales[e0:e0 + n].copy_(s)
        del w32, w
    return out, scales


def gumbel_uniforms(shape: MoEShape) -> np.ndarray:
    """u[T,E] in (0,1): u = (m + 0.5) * 2^-23 with m ~ U{0 .. 2^23-1}.

    m + 0.5 needs at most 24 significant bits, so every u is exactly a float32,
    the smallest is 2^-24 and the largest 1 - 2^-24: never 0 or 1, so
    -log(-log u) is finite without the epsilons of the page's code.
    """
    rng = np.random.Generator(np.random.PCG64(child_seed(shape.seed, "gumbel")))
    m = rng.integers(0, 1 << 23, size=(shape.T, shape.E), dtype=np.int64)
    u = (m.astype(np.float64) + 0.5) * 2.0 ** -23
    u32 = u.astype(np.float32)
    assert np.array_equal(u32.astype(np.float64), u)
    return u32


def zipf_bias(shape: MoEShape) -> np.ndarray:
    """b_e = lambda * ln p_e, p_e proportional to rank_e^-s, ranks a seeded permutation."""
    rng = np.random.Generator(np.random.PCG64(child_seed(shape.seed, "zipf_perm")))
    ranks = rng.permutation(shape.E) + 1
    p = ranks.astype(np.float64) ** (-ZIPF_S)
    p /= p.sum()
    return (ZIPF_LAMBDA * np.log(p)).astype(np.float32)


def make_bias(shape: MoEShape, device="cpu") -> Optional[torch.Tensor]:
    if shape.bias_kind == "none":
        return None
    if shape.bias_kind == "normal0.5":
        # drawn on the host so that CPU and GPU runs share it
        g = torch.Generator(device="cpu")
        g.manual_seed(child_seed(shape.seed, "bias"))
        b = torch.randn(shape.E, generator=g, dtype=torch.float32) * 0.5
        return b.to(device)
    if shape.bias_kind == "zipf1.2":
        return torch.from_numpy(zipf_bias(shape)).to(device)
    raise ValueError(shape.bias_kind)


@dataclasses.dataclass
class MoEInputs:
    shape: MoEShape
    x: torch.Tensor                 # [T,d] f32 or bf16
    w_router: torch.Tensor          # [d,E] f32
    w_gate: torch.Tensor            # [E,F,d] f32 / bf16 / uint8 (e4m3fn codes)
    w_up: torch.Tensor              # [E,F,d]
    w_down: torch.Tensor            # [E,d,F]
    s_gate: Optional[torch.Tensor] = None   # [E,F] f32 (fp8 only)
    s_up: Optional[torch.Tensor] = None     # [E,F]
    s_down: Optional[torch.Tensor] = None   # [E,d]
    sh_gate: Optional[torch.Tensor] = None  # [1,F,d]
    sh_up: Optional[torch.Tensor] = None
    sh_down: Optional[torch.Tensor] = None  # [1,d,F]
    sh_s_gate: Optional[torch.Tensor] = None
    sh_s_up: Optional[torch.Tensor] = None
    sh_s_down: Optional[torch.Tensor] = None
    bias: Optional[torch.Tensor] = None     # [E] f32
    gumbel_u: Optional[torch.Tensor] = None  # [T,E] f32

    def to(self, device) -> "MoEInputs":
        kw = {}
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            kw[f.name] = v.to(device) if isinstance(v, torch.Tensor) else v
        return MoEInputs(**kw)

    def clone_weights(self) -> "MoEInputs":
        """Same values, expert weights (and scales) in freshly allocated memory."""
        kw = {}
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            copy = f.name.startswith(("w_gate", "w_up", "w_down", "s_", "sh_"))
            kw[f.name] = v.clone() if copy and isinstance(v, torch.Tensor) else v
        return MoEInputs(**kw)


def make_inputs(shape: MoEShape, device="cpu", seed: Optional[int] = None) -> MoEInputs:
    """Draw every input of one MoE-layer call for ``shape`` on ``device``."""
    if seed is not None:
        shape = shape.replace(seed=seed)
    T, d, E, F = shape.T, shape.d, shape.E, shape.F
    x = _normal((T, d), 1.0, child_seed(shape.seed, "x"), device)
    if shape.act_dtype == DT_BF16:
        x = x.to(torch.bfloat16)
    w_router = _normal((d, E), 0.02, child_seed(shape.seed, "w_router"), device)
    wg, sg = _expert_tensor(shape, "w_gate", E, F, d, device, shape.w_dtype)
    wu, su = _expert_tensor(shape, "w_up", E, F, d, device, shape.w_dtype)
    wd, sd = _expert_tensor(shape, "w_down", E, d, F, device, shape.w_dtype)
    inp = MoEInputs(shape, x, w_router, wg, wu, wd, sg, su, sd)
    if shape.n_shared:
        inp.sh_gate, inp.sh_s_gate = _expert_tensor(shape, "sh_gate", 1, F, d, device, shape.w_dtype)
        inp.sh_up, inp.sh_s_up = _expert_tensor(shape, "sh_up", 1, F, d, device, shape.w_dtype)
        inp.sh_down, inp.sh_s_down = _expert_tensor(shape, "sh_down", 1, d, F, device, shape.w_dtype)
    inp.bias = make_bias(shape, device)
    if shape.gumbel:
        inp.gumbel_u = torch.from_numpy(gumbel_uniforms(shape)).to(device)
    return inp


def shrink(shape: MoEShape, T: int, d: int, F: int, name: Optional[str] = None) -> MoEShape:
    """Same routing mode and dtypes at smaller sizes (for parity at oracle speed)."""
    return shape.replace(name=name or f"{shape.name}_T{T}_d{d}_F{F}", T=T, d=d, F=F)


def nbytes_of(dtype: int) -> float:
    """Bytes per element (INT4: half a byte; its group words are counted apart)."""
    return {DT_F32: 4, DT_BF16: 2, DT_FP8: 1, DT_INT4: 0.5}[dtype]

