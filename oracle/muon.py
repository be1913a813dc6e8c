"""Muon path in float64, one step at a time.

Sources (page titles and sections):
* OMN "Dual-Manifold Optimization" page - Muon-path paragraphs: momentum-like
  buffer at 0.95, Nesterov-style direction that adds the scaled buffer back to
  the gradient, conversion to fp32, rescale by the largest absolute element
  clamped at 1e-7, Frobenius normalisation with an epsilon, transpose when
  rows exceed columns, five polynomial iterations, orientation restored;
  rectangular-scaling paragraph: sqrt(max(1, m/n)) with m x n the out-by-in
  shape.
* NorMuon paper, section 2.2: eq. (1) M_t = mu M_{t-1} + grad, M_0 = 0;
  eq. (3) W_t = W_{t-1} - eta O_t; eq. (5) X_k = a X + b (X X^T) X +
  c (X X^T)^2 X starting from the Frobenius-normalised momentum.
* NorMuon paper, section 3.1: per-row (per-neuron) mean square of O_t,
  accumulated by an EMA with decay beta2 into v in R^m, then rows normalised
  by it after orthogonalisation.
* MuonClip page, "Newton-Schulz Orthogonalization": the cubic set
  X <- 1.5 X - 0.5 X (X^T X).

* OMN page, Muon-path paragraph: an optional spectral-cap guard on the
  momentum buffer with a power-iteration estimate, inactive by default in
  the recipe.  Its details are not printed; the reading used here: per
  independent matrix, after B_t = mu B_{t-1} + G_t, K power iterations on
  B^T B from v_0 = ones / sqrt(cols) give v_K, sigma = ||B v_K||; when sigma
  exceeds the cap tau the buffer is rescaled to tau / sigma times itself
  (the rescaled buffer is the state and feeds the Nesterov direction).

Readings where the pages are silent (each listed in the design notes):
the Frobenius epsilon is 1e-7 added to the norm; Nesterov uses the updated
buffer, D = G + mu * B_t; NorMuon keeps v_0 = 0, no bias correction, epsilon
outside the square root, and its RMS-matching learning-rate factor is not
applied (the formula is not printed); NorMuon precedes the shape scale;
decoupled weight decay W (1 - lr wd) is available and zero by default.
"""

import math
from typing import Optional, Sequence

import numpy as np

AMAX_FLOOR = 1e-7
FRO_EPS = 1e-7


def momentum(B: np.ndarray, G: np.ndarray, mu: float, nesterov: bool = True):
    """Returns (B_new, D): B_t = mu B_{t-1} + G_t; D = G_t + mu B_t (Nesterov)
    or D = B_t."""
    B_new = mu * B + G
    D = G + mu * B_new if nesterov else B_new.copy()
    return B_new, D


def spectral_estimate(B: np.ndarray, iters: int) -> float:
    """Power-iteration estimate of the largest singular value of B: v_0 =
    ones(cols) / sqrt(cols); v_{k+1} = B^T B v_k / ||B^T B v_k|| for k < iters;
    the estimate is ||B v_iters||.  Zero when B^T B v_k vanishes."""
    B = np.asarray(B, dtype=np.float64)
    v = np.ones(B.shape[1]) / math.sqrt(B.shape[1])
    for _ in range(iters):
        w = B.T @ (B @ v)
        n = math.sqrt(float(np.sum(w * w)))
        if n == 0.0:
            return 0.0
        v = w / n
    return math.sqrt(float(np.sum((B @ v) ** 2)))


def spectral_cap(B: np.ndarray, cap: float, iters: int) -> np.ndarray:
    """The spectral-cap guard on one independent matrix of the buffer:
    B (cap / sigma) when the estimate sigma exceeds cap > 0, else B."""
    if not cap > 0.0:
        return B
    sigma = spectral_estimate(B, iters)
    return B * (cap / sigma) if sigma > cap else B


def normalise(D: np.ndarray) -> np.ndarray:
    """Max-abs rescale (clamped at 1e-7) then Frobenius normalisation."""
    alpha = max(float(np.max(np.abs(D))) if D.size else 0.0, AMAX_FLOOR)
    X = D / alpha
    return X / (math.sqrt(float(np.sum(X * X))) + FRO_EPS)


def newton_schulz(D: np.ndarray, coeffs: Sequence[Sequence[float]]) -> np.ndarray:
    """Orthogonalise one independent matrix (in its stored orientation).

    X_0 is the normalised direction; when rows exceed columns it is transposed
    so that X X^T is formed on the short side.  Each row (a, b, c) of
    ``coeffs`` is one iteration X <- a X + (b A + c A^2) X with A = X X^T.
    The orientation is restored at the end.
    """
    X = normalise(np.asarray(D, dtype=np.float64))
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    for a, b, c in coeffs:
        A = X @ X.T
        X = a * X + (b * A + c * (A @ A)) @ X
    return X.T.copy() if tall else X


def shape_scale(rows: int, cols: int) -> float:
    """sqrt(max(1, m / n)) with m x n the (out, in) shape of the matrix."""
    return math.sqrt(max(1.0, rows / cols))


def normuon_rownorm(O: np.ndarray, v: np.ndarray, beta2: float, eps: float):
    """Per-row second-moment normalisation.  Returns (O_normalised, v_new)."""
    ms = np.mean(O * O, axis=1)
    v_new = beta2 * v + (1.0 - beta2) * ms
    return O / (np.sqrt(v_new)[:, None] + eps), v_new


def apply_update(W: np.ndarray, U: np.ndarray, lr: float, wd: float = 0.0) -> np.ndarray:
    """W <- W (1 - lr wd) - lr U."""
    return W * (1.0 - lr * wd) - lr * U


def muon_param_step(W: np.ndarray, G: np.ndarray, B: np.ndarray, slices,
                    coeffs, lr: float, mu: float, wd: float = 0.0,
                    nesterov: bool = True, normuon_v: Optional[np.ndarray] = None,
                    normuon_beta2: float = 0.95, normuon_eps: float = 1e-8,
                    spectral_cap_value: float = 0.0, spectral_iters: int = 8):
    """One Muon step for one stored weight with its slice table.

    ``slices`` is [(row_offset, rows, cols), ...]; every slice is processed
    independently.  With ``spectral_cap_value`` > 0 each slice of the buffer
    passes the spectral-cap guard before the direction is formed.  Returns
    dict with W, B, D, O (pre-NorMuon NS output laid out like W), U (final
    scaled update) and v (NorMuon state or None).
    """
    B_new, D = momentum(B, G, mu, nesterov)
    if spectral_cap_value > 0.0:
        for off, r, _ in slices:
            B_new[off:off + r] = spectral_cap(B_new[off:off + r], spectral_cap_value,
                                              spectral_iters)
        D = G + mu * B_new if nesterov else B_new.copy()
    O = np.zeros_like(D)
    U = np.zeros_like(D)
    v_new = None if normuon_v is None else normuon_v.copy()
    for off, r, c in slices:
        Os = newton_schulz(D[off:off + r], coeffs)
        O[off:off + r] = Os
        if v_new is not None:
            Os, v_new[off:off + r] = normuon_rownorm(Os, normuon_v[off:off + r],
                                                     normuon_beta2, normuon_eps)
        U[off:off + r] = shape_scale(r, c) * Os
    return {"W": apply_update(W, U, lr, wd), "B": B_new, "D": D, "O": O, "U": U,
            "v": v_new}
