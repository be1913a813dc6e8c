"""Pins of the oracle's spectral-cap guard (OMN "Dual-Manifold Optimization"
page, Muon-path paragraph: an optional guard with a power-iteration estimate
of the buffer's spectral norm, inactive by default).  The page prints no
formula; the reading pinned here is K power iterations on B^T B from
v_0 = ones / sqrt(cols), the estimate ||B v_K||, and B rescaled to the cap
when the estimate exceeds it, per independent matrix.

None of the pins re-types the iteration: the closed form follows from the
singular value decomposition, the others from invariants."""

import math

import numpy as np
import pytest

import workloads as wl
from oracle import muon


def _prescribed(r, c, sig, seed):
    g = np.random.default_rng(seed)
    s = min(r, c)
    U, _ = np.linalg.qr(g.standard_normal((r, s)))
    V, _ = np.linalg.qr(g.standard_normal((c, s)))
    return (U * sig) @ V.T, V


@pytest.mark.parametrize("shape", [(12, 7), (7, 12), (30, 30)])
@pytest.mark.parametrize("iters", [1, 2, 5, 9])
def test_estimate_closed_form_from_the_svd(shape, iters):
    """With B = U diag(s) V^T and a = V^T v_0, (B^T B)^K v_0 = V diag(s^2K) a,
    so the estimate squared is sum a^2 s^(4K+2) / sum a^2 s^(4K)."""
    r, c = shape
    sig = np.linspace(1.7, 0.3, min(r, c))
    B, V = _prescribed(r, c, sig, 5)
    a = V.T @ (np.ones(c) / math.sqrt(c))
    want = math.sqrt(np.sum(a ** 2 * sig ** (4 * iters + 2)) / np.sum(a ** 2 * sig ** (4 * iters)))
    assert muon.spectral_estimate(B, iters) == pytest.approx(want, rel=1e-12)


def test_estimate_without_iterations_is_the_start_vector_image():
    B, V = _prescribed(9, 6, np.array([3.0, 2.0, 1.0, 0.5, 0.2, 0.1]), 6)
    a = V.T @ (np.ones(6) / math.sqrt(6))
    assert muon.spectral_estimate(B, 0) == pytest.approx(math.sqrt(np.sum(a ** 2 * np.array(
        [3.0, 2.0, 1.0, 0.5, 0.2, 0.1]) ** 2)), rel=1e-12)


def test_rank_one_is_exact_after_one_iteration():
    g = np.random.default_rng(7)
    x, y = g.standard_normal(11), g.standard_normal(5)
    B = 2.5 * np.outer(x / np.linalg.norm(x), y / np.linalg.norm(y))
    for k in (1, 3, 8):
        assert muon.spectral_estimate(B, k) == pytest.approx(2.5, rel=1e-13)


def test_converges_to_the_spectral_norm_and_never_exceeds_it():
    g = np.random.default_rng(8)
    for shape in ((40, 25), (25, 40)):
        B = g.standard_normal(shape)
        top = np.linalg.norm(B, 2)
        prev = 0.0
        for k in (1, 2, 4, 8, 16):
            est = muon.spectral_estimate(B, k)
            assert est <= top * (1 + 1e-12)          # a Rayleigh quotient
            assert est >= prev * (1 - 1e-12)         # monotone for power iteration
            prev = est
    B, _ = _prescribed(30, 20, np.geomspace(4.0, 0.1, 20), 9)   # gap 4 -> 3.4
    assert muon.spectral_estimate(B, 200) == pytest.approx(4.0, rel=1e-12)


def test_zero_matrix_estimate_is_zero():
    assert muon.spectral_estimate(np.zeros((4, 6)), 5) == 0.0
    np.testing.assert_array_equal(muon.spectral_cap(np.zeros((4, 6)), 1.0, 5), 0.0)


def test_cap_rescales_to_the_cap_only_above_it():
    g = np.random.default_rng(10)
    B = g.standard_normal((16, 24))
    est = muon.spectral_estimate(B, 6)
    # above the cap: the estimate of the capped buffer is the cap (the
    # estimate is positively homogeneous), and the direction is unchanged
    capped = muon.spectral_cap(B, 0.5 * est, 6)
    assert muon.spectral_estimate(capped, 6) == pytest.approx(0.5 * est, rel=1e-12)
    np.testing.assert_allclose(capped, B * 0.5, rtol=1e-12)
    # at or below the cap, and with the guard off: untouched
    for cap in (est * 1.0000001, 10 * est, 0.0, -1.0):
        assert muon.spectral_cap(B, cap, 6) is B


def test_step_applies_the_cap_per_slice_before_the_direction():
    """In a Muon step the cap acts on each independent matrix of the buffer
    (views as in the kimi-k3 layout declarations) and the Nesterov direction
    is formed from the capped buffer: slices stay independent, an inactive
    guard gives the plain step, and a capped slice's buffer has estimate tau."""
    g = np.random.default_rng(11)
    W = g.standard_normal((12, 8)) * 0.02
    G = g.standard_normal((12, 8))
    B0 = g.standard_normal((12, 8))
    slices = [(0, 4, 8), (4, 8, 8)]
    cf = wl.coeff_table("cubic")
    plain = muon.muon_param_step(W, G, B0, slices, cf, 0.01, 0.95)
    off = muon.muon_param_step(W, G, B0, slices, cf, 0.01, 0.95, spectral_cap_value=0.0)
    np.testing.assert_array_equal(plain["B"], off["B"])
    est = [muon.spectral_estimate(plain["B"][o:o + r], 8) for o, r, _ in slices]
    tau = 0.5 * min(est)
    capped = muon.muon_param_step(W, G, B0, slices, cf, 0.01, 0.95, spectral_cap_value=tau)
    for (o, r, _), e in zip(slices, est):
        Bs = capped["B"][o:o + r]
        np.testing.assert_allclose(Bs, plain["B"][o:o + r] * (tau / e), rtol=1e-12)
        assert muon.spectral_estimate(Bs, 8) == pytest.approx(tau, rel=1e-12)
    np.testing.assert_allclose(capped["D"], G + 0.95 * capped["B"], rtol=1e-14)
    # slice independence: changing slice 1's gradient leaves slice 0 alone
    G2 = G.copy()
    G2[4:] *= -3.0
    other = muon.muon_param_step(W, G2, B0, slices, cf, 0.01, 0.95, spectral_cap_value=tau)
    np.testing.assert_array_equal(other["B"][:4], capped["B"][:4])


# -- planted mistakes: each must trip at least one pin above ------------------

def _mutant_random_start(B, iters):
    B = np.asarray(B, dtype=np.float64)
    v = np.random.default_rng(0).standard_normal(B.shape[1])
    v /= np.linalg.norm(v)
    for _ in range(iters):
        w = B.T @ (B @ v)
        v = w / np.linalg.norm(w)
    return float(np.linalg.norm(B @ v))


def _mutant_squared(B, iters):       # reports ||B^T B v|| instead of ||B v||
    B = np.asarray(B, dtype=np.float64)
    v = np.ones(B.shape[1]) / math.sqrt(B.shape[1])
    for _ in range(iters):
        w = B.T @ (B @ v)
        v = w / np.linalg.norm(w)
    return float(np.linalg.norm(B.T @ (B @ v)))


def _mutant_off_by_one(B, iters):    # one iteration fewer
    B = np.asarray(B, dtype=np.float64)
    v = np.ones(B.shape[1]) / math.sqrt(B.shape[1])
    for _ in range(max(iters - 1, 0)):
        w = B.T @ (B @ v)
        v = w / np.linalg.norm(w)
    return float(np.linalg.norm(B @ v))


@pytest.mark.parametrize("mutant", [_mutant_random_start, _mutant_squared, _mutant_off_by_one])
def test_planted_estimate_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(muon, "spectral_estimate", mutant)
    failed = 0
    for shape in ((12, 7), (7, 12), (30, 30)):
        for iters in (1, 2, 5, 9):
            try:
                test_estimate_closed_form_from_the_svd(shape, iters)
            except AssertionError:
                failed += 1
    assert failed > 0
