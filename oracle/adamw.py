"""AdamW path with a global-norm clip over the AdamW parameters, in float64.

Sources: OMN "Dual-Manifold Optimization" page, recipe paragraph (betas
(0.90, 0.95), epsilon 1e-8, clipping at 1.0 on AdamW parameters only, Muon
never clipped, zero decay); Qwen3.8 optimizer notes, background on Adam
(first and second moments with bias correction) and AdamW (weight decay
decoupled from the adaptive step).

Readings: the clip factor is max_norm / T when T > max_norm and 1 otherwise,
with no epsilon; epsilon is added outside the square root of the corrected
second moment; decay multiplies the pre-update weight; t counts per parameter
and starts at 1.
"""

import math
from typing import Sequence

import numpy as np


def global_norm(grads: Sequence[np.ndarray]) -> float:
    """T = sqrt(sum over all given gradients of g^2)."""
    s = 0.0
    for g in grads:
        if g is not None:
            s += float(np.sum(np.asarray(g, dtype=np.float64) ** 2))
    return math.sqrt(s)


def clip_factor(total_norm: float, max_norm: float) -> float:
    return max_norm / total_norm if total_norm > max_norm else 1.0


def adamw_update(W, G, m, v, t: int, lr: float, beta1: float, beta2: float,
                 eps: float, wd: float, kappa: float = 1.0):
    """One AdamW step on one parameter; returns (W, m, v)."""
    g = kappa * G
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    W = W * (1.0 - lr * wd) - lr * m_hat / (np.sqrt(v_hat) + eps)
    return W, m, v


def adamw_clip_step(params, lr, beta1, beta2, eps, wd, max_norm):
    """Joint clipped AdamW step.  ``params``: list of dicts with W, G (None =
    skip), m, v, t (the step number to use, >= 1) and optionally wd (overrides
    the shared ``wd``).  Returns (list of updated (W, m, v) or None for
    skipped params, T, kappa)."""
    T = global_norm([p["G"] for p in params])
    kappa = clip_factor(T, max_norm)
    out = []
    for p in params:
        if p["G"] is None:
            out.append(None)
            continue
        out.append(adamw_update(p["W"], p["G"], p["m"], p["v"], p["t"], lr,
                                beta1, beta2, eps, p.get("wd", wd), kappa))
    return out, T, kappa
