"""Pins for the oracle's Muon path (CPU only).

Each pin is fixed by the pages or by mathematics, not by re-running the
oracle's own formula: closed forms (momentum with a constant gradient, the
prescribed-SVD scalar recurrence), the SVD polar factor, the pages' diag(100,1)
example, degenerate inputs, invariants (transpose, scale, slice independence)
and the NorMuon value for exactly orthogonal rows.
"""

import json
import math
import os

import numpy as np
import pytest

import workloads as wl
from oracle import muon, views

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
CUBIC = wl.coeff_table("cubic")
QUINTIC = wl.coeff_table("quintic")


def _orth(rng, n, k):
    q, _ = np.linalg.qr(rng.standard_normal((n, k)))
    return q


def _scalar_ns(sig, coeffs):
    """The NS polynomial acting on one singular value, p(x) = a x + b x^3 + c x^5."""
    x = np.array(sig, dtype=np.float64)
    for a, b, c in coeffs:
        x = a * x + b * x ** 3 + c * x ** 5
    return x


# --- momentum -------------------------------------------------------------

def test_momentum_constant_gradient_closed_form():
    # D_t / G = 1 + mu (1 - mu^t) / (1 - mu) for a constant G (NorMuon eq. (1),
    # Nesterov reading D = G + mu B_t).
    G = np.full((3, 4), 0.7)
    B = np.zeros_like(G)
    for t, want in zip((1, 2, 3), (1.95, 2.8525, 3.709875)):
        B, D = muon.momentum(B, G, 0.95)
        np.testing.assert_allclose(D / G, want, rtol=0, atol=1e-14)
        np.testing.assert_allclose(B / G, (1 - 0.95 ** t) / 0.05, rtol=1e-14)


def test_momentum_without_nesterov_is_buffer():
    G = np.arange(6.0).reshape(2, 3)
    B, D = muon.momentum(np.ones((2, 3)), G, 0.9, nesterov=False)
    np.testing.assert_array_equal(B, 0.9 + G)
    np.testing.assert_array_equal(D, B)


# --- normalisation ----------------------------------------------------------

def test_normalise_unit_frobenius_and_scale_invariant():
    rng = np.random.default_rng(0)
    D = rng.standard_normal((5, 7)) * 1e-3
    X = muon.normalise(D)
    assert abs(np.linalg.norm(X) - 1.0) < 1e-6
    for c in (1e-2, 3.0, 1e4):          # amax stays above the 1e-7 floor
        np.testing.assert_allclose(muon.normalise(c * D), X, atol=1e-6)


def test_normalise_amax_floor():
    # below the floor, alpha = 1e-7 and the Frobenius epsilon is no longer
    # negligible: X = D / (||D|| + 1e-7 * 1e-7).
    D = np.array([[3e-9, -4e-9]])
    want = D / (5e-9 + 1e-14)
    np.testing.assert_allclose(muon.normalise(D), want, rtol=1e-12)


def test_normalise_zero_is_zero():
    X = muon.normalise(np.zeros((3, 4)))
    assert np.all(X == 0) and np.all(np.isfinite(X))


# --- Newton-Schulz ----------------------------------------------------------

@pytest.mark.parametrize("shape", [(6, 6), (4, 9), (11, 3)])
@pytest.mark.parametrize("kind", ["cubic", "quintic"])
def test_ns_prescribed_svd_closed_form(shape, kind):
    # D = U diag(s) V^T  =>  X_N = U diag(p_N o ... o p_1(s_hat)) V^T with
    # s_hat the normalised singular values (NorMuon eqs. (4)-(5)).
    m, n = shape
    k = min(m, n)
    rng = np.random.default_rng(m * 31 + n)
    U, V = _orth(rng, m, k), _orth(rng, n, k)
    s = np.linspace(1.0, 0.05, k) * rng.uniform(0.5, 2.0)
    D = U @ np.diag(s) @ V.T
    alpha = np.max(np.abs(D))
    s_hat = s / (np.sqrt(np.sum(s ** 2)) + alpha * 1e-7)
    coeffs = wl.coeff_table(kind)
    want = U @ np.diag(_scalar_ns(s_hat, coeffs)) @ V.T
    got = muon.newton_schulz(D, coeffs)
    assert got.shape == D.shape
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_ns_per_step_coefficient_rows_are_used_in_order():
    rng = np.random.default_rng(5)
    U, V = _orth(rng, 5, 5), _orth(rng, 5, 5)
    s = np.array([1.0, 0.6, 0.3, 0.1, 0.02])
    D = U @ np.diag(s) @ V.T
    table = np.array([[2.0, -1.5, 0.5], [1.5, -0.5, 0.0], [15 / 8, -10 / 8, 3 / 8]])
    s_hat = s / (np.linalg.norm(s) + np.max(np.abs(D)) * 1e-7)
    want = U @ np.diag(_scalar_ns(s_hat, table)) @ V.T
    np.testing.assert_allclose(muon.newton_schulz(D, table), want, atol=1e-12)
    rev = U @ np.diag(_scalar_ns(s_hat, table[::-1])) @ V.T
    assert np.abs(muon.newton_schulz(D, table) - rev).max() > 1e-6


def test_diag100_example_from_page():
    gold = json.load(open(os.path.join(GOLDEN, "diag100.json")))
    D = np.array(gold["input"])
    polar = np.array(gold["polar_factor"])
    # converged: the cubic needs ~16 steps, the quintic ~11, from s2 = 0.01
    np.testing.assert_allclose(muon.newton_schulz(D, wl.coeff_table("cubic", 20)), polar,
                               atol=1e-12)
    np.testing.assert_allclose(muon.newton_schulz(D, wl.coeff_table("quintic", 14)), polar,
                               atol=1e-12)
    # five steps: diagonal, s1 at its fixed point, s2 from the scalar recurrence
    s_hat = np.array([100.0, 1.0]) / (math.sqrt(10001.0) + 100.0 * 1e-7)
    for kind in ("cubic", "quintic"):
        X = muon.newton_schulz(D, wl.coeff_table(kind))
        want = _scalar_ns(s_hat, wl.coeff_table(kind))
        np.testing.assert_allclose(np.diag(X), want, atol=1e-13)
        assert abs(X[0, 1]) < 1e-15 and abs(X[1, 0]) < 1e-15
        assert abs(X[0, 0] - 1.0) < 1e-9 and 0.05 < X[1, 1] < 0.3   # not yet converged


@pytest.mark.parametrize("shape", [(8, 8), (12, 5), (5, 12)])
def test_ns_converges_to_svd_polar_factor(shape):
    rng = np.random.default_rng(shape[0] * 7 + shape[1])
    m, n = shape
    k = min(m, n)
    U, V = _orth(rng, m, k), _orth(rng, n, k)
    s = rng.uniform(0.3, 1.0, k)       # well conditioned
    D = U @ np.diag(s) @ V.T
    u, _, vt = np.linalg.svd(D, full_matrices=False)
    got = muon.newton_schulz(D, wl.coeff_table("cubic", 40))
    np.testing.assert_allclose(got, u @ vt, atol=1e-10)


@pytest.mark.parametrize("shape", [(9, 1), (1, 9), (6, 4)])
def test_rank_one_maps_to_normalised_input(shape):
    # A rank-1 slice is not zeroed: its single singular value sits at the
    # fixed point 1 of p (p(1) = a + b + c = 1).
    rng = np.random.default_rng(11)
    u = rng.standard_normal((shape[0], 1))
    v = rng.standard_normal((1, shape[1]))
    D = u @ v
    for coeffs in (CUBIC, QUINTIC):
        got = muon.newton_schulz(D, coeffs)
        np.testing.assert_allclose(got, D / np.linalg.norm(D), atol=1e-12)


def test_zero_slice_gives_zero():
    got = muon.newton_schulz(np.zeros((4, 6)), CUBIC)
    assert np.all(got == 0)


def test_transpose_equivalence():
    rng = np.random.default_rng(3)
    D = rng.standard_normal((7, 13))
    np.testing.assert_allclose(muon.newton_schulz(D.T, QUINTIC), muon.newton_schulz(D, QUINTIC).T,
                               atol=1e-14)


def test_quintic_coefficients_are_second_order():
    a, b, c = wl.QUINTIC
    assert a + b + c == 1.0               # p(1) = 1
    assert a + 3 * b + 5 * c == 0.0       # p'(1) = 0
    assert 6 * b + 20 * c == 0.0          # p''(1) = 0
    a, b, c = wl.CUBIC
    assert a + b + c == 1.0 and a + 3 * b + 5 * c == 0.0


# --- shape scale, NorMuon, update ------------------------------------------

def test_shape_scale_values():
    assert muon.shape_scale(5632, 2048) == pytest.approx(1.6583123951777, abs=1e-12)
    assert muon.shape_scale(4096, 1024) == 2.0
    assert muon.shape_scale(5504, 2048) == pytest.approx(1.6393596310755, abs=1e-12)
    assert muon.shape_scale(128, 4096) == 1.0 and muon.shape_scale(2048, 2048) == 1.0


def test_normuon_on_exactly_orthogonal_rows():
    rng = np.random.default_rng(2)
    r, c = 4, 10
    O = _orth(rng, c, r).T        # r orthonormal rows: mean square = 1 / c
    v0 = np.zeros(r)
    On, v1 = muon.normuon_rownorm(O, v0, 0.95, 1e-8)
    np.testing.assert_allclose(v1, 0.05 / c, rtol=1e-14)
    np.testing.assert_allclose(On, O / (math.sqrt(0.05 / c) + 1e-8), rtol=1e-13)


def test_normuon_rows_independent_and_ema():
    O = np.array([[3.0, 4.0], [0.0, 0.0]])
    On, v = muon.normuon_rownorm(O, np.array([2.0, 1.0]), 0.5, 0.0)
    np.testing.assert_allclose(v, [0.5 * 2 + 0.5 * 12.5, 0.5])
    np.testing.assert_allclose(On[0], O[0] / math.sqrt(v[0]))
    assert np.all(On[1] == 0)


def test_update_is_decoupled_decay_then_step():
    W = np.array([[1.0, -2.0]])
    U = np.array([[0.5, 0.25]])
    np.testing.assert_allclose(muon.apply_update(W, U, 0.1, 0.5),
                               W * 0.95 - 0.1 * U)


# --- whole-weight invariants --------------------------------------------------

def test_slice_independence():
    rng = np.random.default_rng(4)
    shape = (20, 8)
    sl = views.expand(shape, (2, 10, 8), (4, 6))
    W = rng.standard_normal(shape)
    G = rng.standard_normal(shape)
    base = muon.muon_param_step(W, G, np.zeros(shape), sl, CUBIC, 0.01, 0.95)
    G2 = G.copy()
    G2[4:10] *= -3.0                     # slice 1 only
    pert = muon.muon_param_step(W, G2, np.zeros(shape), sl, CUBIC, 0.01, 0.95)
    changed = ~np.all(base["W"] == pert["W"], axis=1)
    assert np.array_equal(np.nonzero(changed)[0], np.arange(4, 10))


def test_fused_gate_up_equals_separate_matrices():
    rng = np.random.default_rng(8)
    I, C = 12, 5
    W = rng.standard_normal((2 * I, C))
    G = rng.standard_normal((2 * I, C))
    fused = muon.muon_param_step(W, G, np.zeros_like(W), views.expand(W.shape, (2, I, C)),
                                 CUBIC, 0.01, 0.95, normuon_v=np.zeros(2 * I))
    for h in range(2):
        rows = slice(h * I, (h + 1) * I)
        sep = muon.muon_param_step(W[rows], G[rows], np.zeros((I, C)), [(0, I, C)], CUBIC,
                                   0.01, 0.95, normuon_v=np.zeros(I))
        assert np.array_equal(fused["W"][rows], sep["W"])
        assert np.array_equal(fused["v"][rows], sep["v"])


def test_tall_slice_scale_applied():
    rng = np.random.default_rng(9)
    W = np.zeros((8, 2))
    G = rng.standard_normal((8, 2))
    out = muon.muon_param_step(W, G, np.zeros_like(G), [(0, 8, 2)], CUBIC, 1.0, 0.95)
    np.testing.assert_allclose(out["U"], 2.0 * out["O"])
    np.testing.assert_allclose(out["W"], -out["U"])


def test_state_sizes():
    # Muon keeps m*n momentum floats; NorMuon adds m; AdamW keeps 2*m*n.
    from oracle.hybrid import HybridState, HyperParams, hybrid_step
    descs = [{"name": "w", "shape": (6, 4), "dtype": "f32"},
             {"name": "e", "shape": (6, 4), "role": "embedding", "no_decay": True, "dtype": "f32"}]
    rng = np.random.default_rng(1)
    W = {d["name"]: rng.standard_normal(d["shape"]) for d in descs}
    G = {d["name"]: rng.standard_normal(d["shape"]) for d in descs}
    st = HybridState()
    hybrid_step(descs, W, G, st, HyperParams(normuon=True))
    assert st.B["w"].size == 24 and st.nv["w"].size == 6
    assert st.m["e"].size + st.v["e"].size == 48 and "e" not in st.B
