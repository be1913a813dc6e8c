"""Pins for the oracle's AdamW path and clip (CPU only)."""

import math

import numpy as np
import pytest

import workloads as wl
from oracle import adamw, bf16


def test_first_step_is_sign_like():
    # t = 1: m_hat = g and v_hat = g^2, so dW = -lr g / (|g| + eps).
    g = np.array([0.3, -2.0, 1e-9, 0.0])
    W0 = np.array([1.0, 1.0, 1.0, 1.0])
    W, m, v = adamw.adamw_update(W0, g, np.zeros(4), np.zeros(4), 1, 1e-3, 0.9, 0.95, 1e-8, 0.0)
    np.testing.assert_allclose(W - W0, -1e-3 * g / (np.abs(g) + 1e-8), rtol=1e-10, atol=1e-18)
    np.testing.assert_allclose(m, 0.1 * g, rtol=1e-15)
    np.testing.assert_allclose(v, 0.05 * g * g, rtol=1e-15)


def test_constant_gradient_same_step_every_time():
    g = np.array([0.5, -0.25])
    W, m, v = np.zeros(2), np.zeros(2), np.zeros(2)
    prev = None
    for t in range(1, 6):
        W1, m, v = adamw.adamw_update(W, g, m, v, t, 0.01, 0.9, 0.95, 1e-8, 0.0)
        step = W1 - W
        np.testing.assert_allclose(step, -0.01 * g / (np.abs(g) + 1e-8), rtol=1e-12)
        W = W1


def test_decoupled_decay():
    # decay shrinks W directly; it does not pass through the adaptive step.
    W, _, _ = adamw.adamw_update(np.array([2.0]), np.array([0.0]), np.zeros(1), np.zeros(1), 1,
                                 0.1, 0.9, 0.95, 1e-8, 0.5)
    assert W[0] == pytest.approx(2.0 * 0.95)
    W, _, _ = adamw.adamw_update(np.array([2.0]), np.array([0.5]), np.zeros(1), np.zeros(1), 1,
                                 0.1, 0.9, 0.95, 1e-8, 0.5)
    assert W[0] == pytest.approx(2.0 * 0.95 - 0.1 * 0.5 / (0.5 + 1e-8), abs=1e-15)


def test_clip_active_gives_unit_norm():
    rng = np.random.default_rng(0)
    gs = [rng.standard_normal(50), rng.standard_normal((4, 5))]
    T = adamw.global_norm(gs)
    assert T == pytest.approx(math.sqrt(sum(np.sum(g ** 2) for g in gs)))
    k = adamw.clip_factor(T, 1.0)
    assert math.isclose(math.sqrt(sum(np.sum((k * g) ** 2) for g in gs)), 1.0, rel_tol=1e-14)


def test_clip_inactive_and_skipped_grads():
    assert adamw.clip_factor(0.7, 1.0) == 1.0
    assert adamw.clip_factor(1.0, 1.0) == 1.0
    items = [{"W": np.ones(3), "G": None, "m": np.zeros(3), "v": np.zeros(3), "t": 1},
             {"W": np.ones(2), "G": np.array([3.0, 4.0]), "m": np.zeros(2), "v": np.zeros(2),
              "t": 1}]
    out, T, k = adamw.adamw_clip_step(items, 1e-3, 0.9, 0.95, 1e-8, 0.0, 1.0)
    assert out[0] is None and T == 5.0 and k == 0.2
    np.testing.assert_allclose(out[1][1], 0.1 * 0.2 * np.array([3.0, 4.0]))


def test_bias_correction_second_step():
    # two steps, hand expanded: m2 = 0.9*0.1 g1 + 0.1 g2, v2 likewise with 0.95.
    g1, g2 = 0.2, -0.6
    W, m, v = adamw.adamw_update(np.array([0.0]), np.array([g1]), np.zeros(1), np.zeros(1), 1,
                                 1.0, 0.9, 0.95, 0.0, 0.0)
    W, m, v = adamw.adamw_update(W, np.array([g2]), m, v, 2, 1.0, 0.9, 0.95, 0.0, 0.0)
    m2 = 0.09 * g1 + 0.1 * g2
    v2 = 0.95 * 0.05 * g1 ** 2 + 0.05 * g2 ** 2
    step2 = -(m2 / (1 - 0.81)) / math.sqrt(v2 / (1 - 0.9025))
    assert W[0] == pytest.approx(-g1 / abs(g1) + step2, abs=1e-14)


def test_bf16_rounding_matches_bit_codec():
    # two independent implementations: frexp/rint (oracle) vs integer bit
    # trick (input codec) must agree on every fp32 value.
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(
        -30, 30, 20000), np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -1 - 2 ** -8, 0.0, -0.0,
                                   3.3895e38, 1e-40], dtype=np.float32)]).astype(np.float32)
    want = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(x)).astype(np.float64)
    got = bf16.round_bf16(x.astype(np.float64))
    assert np.array_equal(np.isinf(got), np.isinf(want))
    fin = np.isfinite(want)
    assert np.array_equal(got[fin], want[fin])
    assert bf16.round_bf16(np.array([1 + 2 ** -8]))[0] == 1.0        # tie to even
    assert bf16.round_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6


def test_widen_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0001, 0x7F7F], dtype=np.uint16)
    np.testing.assert_array_equal(bf16.widen(bits, "bf16"),
                                  [1.0, -1.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127])
