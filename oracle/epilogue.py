"""fp64 oracle of the attention block's output epilogue (test infrastructure
only; numpy, CPU).

Source, cited by page title and section:
  [KDA-blog] "Kimi k3 技术报告详解（1）——架构再升华", section "Gated MLA",
             output equation: the block output is W_o applied to
             Sigmoid(W_g x_t) elementwise-times RMSNorm(o~_t).

Only the part before the weight product W_o is computed here; the gate
logits W_g x_t are an input. Readings of what the equation leaves open:
RMSNorm normalises each head's d_v outputs by the root of their mean square
plus eps (eps = 1e-6 unless given) and multiplies by an optional per-channel
weight of length d_v (ones when absent).
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def oracle_gated_rmsnorm(o, gate_logits, weight: Optional[object] = None,
                         eps: float = 1e-6) -> np.ndarray:
    """y = sigmoid(gate_logits) * o / sqrt(mean(o^2 over the last axis) + eps) * weight.

    o, gate_logits: [..., Dv]; weight: [Dv] or None. Returns float64 [..., Dv].
    """
    o64 = _f64(o)
    z64 = _f64(gate_logits)
    if o64.shape != z64.shape:
        raise ValueError("o and gate_logits must have the same shape")
    mean_sq = np.mean(o64 * o64, axis=-1, keepdims=True)
    normed = o64 / np.sqrt(mean_sq + eps)
    if weight is not None:
        normed = normed * _f64(weight)
    with np.errstate(over="ignore"):  # exp(-z) = inf for z << 0 gives the limit 0
        gate = 1.0 / (1.0 + np.exp(-z64))
    return gate * normed
