// Selection key and gate-weight basis of one (token, expert), shared by the
// router's top-k and the load-balancing statistics so both see the same values.
//
// softmax scoring (page "GPT-4 has 1.8T parameters but uses 2% per token"
// (mlqm.cn), s3.1 gating network: Gumbel noise and temperature before the
// softmax; page "Parameter scale and the truth about sparse activation"
// (deepseek.csdn.net), s3.1 temperature):
//     l = z (+ b for a logit bias) (+ g, g = -log(-log u)) / tau
//     key = l, or l + b for a selection-only bias; basis = l
// sigmoid scoring (page "From sparse MoE to conditional memory" (m.nxbn.cn),
// per-expert bias steering the selection):
//     s = sigmoid(z); key = s, or s + b; basis = s
// Every step is one float32 operation in this order (g and the sigmoid are
// computed in float64 and rounded once), so the result is reproducible.
#pragma once

#include "common.h"

namespace moe {

struct KeyBasis {
  float key;
  float basis;
};

__device__ __forceinline__ KeyBasis key_basis(float z, int e, size_t te, int score, int bias_mode,
                                              const float* __restrict__ bias, const float* __restrict__ gumbel_u,
                                              float tau) {
  KeyBasis r;
  if (score == MOE_SCORE_SOFTMAX) {
    float l = z;
    if (bias_mode == MOE_BIAS_LOGIT) l = l + bias[e];
    if (gumbel_u) {
      const double u = (double)gumbel_u[te];
      l = l + (float)(-log(-log(u)));
    }
    l = l / tau;
    r.basis = l;
    r.key = (bias_mode == MOE_BIAS_SELECT_ONLY) ? l + bias[e] : l;
  } else {
    const float s = (float)(1.0 / (1.0 + exp(-(double)z)));
    r.basis = s;
    r.key = (bias_mode == MOE_BIAS_SELECT_ONLY) ? s + bias[e] : s;
  }
  return r;
}

}  // namespace moe
