"""Planted-mistake check: each plausible slip in the oracle trips a pin.

Mutants are planted in the oracle on the CPU with monkeypatch; the pin tests
are then run against the mutated oracle and at least one must fail.
"""

import math

import numpy as np
import pytest

from oracle import adamw, muon, views

import test_oracle_adamw as TA
import test_oracle_muon as TM
import test_oracle_views_routing as TV


def _ns_mutant(kind):
    def ns(D, coeffs):
        X = muon.normalise(np.asarray(D, dtype=np.float64)) if kind != "no_norm" else D / np.abs(
            D).max()
        tall = X.shape[0] > X.shape[1]
        if tall:
            X = X.T
        rows = coeffs[::-1] if kind == "reversed" else coeffs
        for a, b, c in rows:
            A = X @ X.T
            if kind == "drop_c":
                X = a * X + b * A @ X
            elif kind == "sign_b":
                X = a * X - b * A @ X + c * (A @ A) @ X
            elif kind == "square_not_cubed":
                X = a * X + (b * A + c * A) @ X
            else:
                X = a * X + (b * A + c * (A @ A)) @ X
        if tall and kind != "no_untranspose":
            X = X.T
        return X.copy()
    return ns


NS_PINS = [
    lambda: [TM.test_ns_prescribed_svd_closed_form(s, k) for s in [(6, 6), (4, 9), (11, 3)]
             for k in ("cubic", "quintic")],
    TM.test_ns_per_step_coefficient_rows_are_used_in_order,
    TM.test_diag100_example_from_page,
    lambda: [TM.test_ns_converges_to_svd_polar_factor(s) for s in [(8, 8), (12, 5), (5, 12)]],
    lambda: [TM.test_rank_one_maps_to_normalised_input(s) for s in [(9, 1), (1, 9), (6, 4)]],
    TM.test_transpose_equivalence,
]


def _some_pin_fails(pins):
    for p in pins:
        try:
            p()
        except (AssertionError, ValueError):
            return True
    return False


@pytest.mark.parametrize("kind", ["drop_c", "sign_b", "square_not_cubed", "reversed",
                                  "no_norm", "no_untranspose"])
def test_ns_mutants_are_caught(monkeypatch, kind):
    monkeypatch.setattr(muon, "newton_schulz", _ns_mutant(kind))
    assert _some_pin_fails(NS_PINS)


def test_momentum_mutants_are_caught(monkeypatch):
    def old_buffer(B, G, mu, nesterov=True):
        return mu * B + G, G + mu * B          # Nesterov with the previous buffer

    def ema(B, G, mu, nesterov=True):
        Bn = mu * B + (1 - mu) * G
        return Bn, G + mu * Bn
    for m in (old_buffer, ema):
        monkeypatch.setattr(muon, "momentum", m)
        assert _some_pin_fails([TM.test_momentum_constant_gradient_closed_form])


def test_normuon_mutants_are_caught(monkeypatch):
    def cols(O, v, beta2, eps):
        ms = np.mean(O * O, axis=0)[: O.shape[0]]
        vn = beta2 * v + (1 - beta2) * ms
        return O / (np.sqrt(vn)[:, None] + eps), vn

    def eps_inside(O, v, beta2, eps):
        vn = beta2 * v + (1 - beta2) * np.mean(O * O, axis=1)
        return O / np.sqrt(vn + eps)[:, None], vn
    for m in (cols, eps_inside):
        monkeypatch.setattr(muon, "normuon_rownorm", m)
        assert _some_pin_fails([TM.test_normuon_on_exactly_orthogonal_rows,
                                TM.test_normuon_rows_independent_and_ema])


def test_adamw_mutants_are_caught(monkeypatch):
    orig = adamw.adamw_update

    def no_bias(W, G, m, v, t, lr, b1, b2, eps, wd, kappa=1.0):
        g = kappa * G
        m = b1 * m + (1 - b1) * g
        v = b2 * v + (1 - b2) * g * g
        return W * (1 - lr * wd) - lr * m / (np.sqrt(v) + eps), m, v

    def eps_inside(W, G, m, v, t, lr, b1, b2, eps, wd, kappa=1.0):
        g = kappa * G
        m = b1 * m + (1 - b1) * g
        v = b2 * v + (1 - b2) * g * g
        mh, vh = m / (1 - b1 ** t), v / (1 - b2 ** t)
        return W * (1 - lr * wd) - lr * mh / np.sqrt(vh + eps), m, v

    def coupled_decay(W, G, m, v, t, lr, b1, b2, eps, wd, kappa=1.0):
        return orig(W, G + wd * W, m, v, t, lr, b1, b2, eps, 0.0, kappa)
    pins = [TA.test_first_step_is_sign_like, TA.test_constant_gradient_same_step_every_time,
            TA.test_decoupled_decay, TA.test_bias_correction_second_step]
    for m in (no_bias, eps_inside, coupled_decay):
        monkeypatch.setattr(adamw, "adamw_update", m)
        assert _some_pin_fails(pins)
    monkeypatch.setattr(adamw, "adamw_update", orig)
    monkeypatch.setattr(adamw, "clip_factor", lambda T, mx: mx / T)
    assert _some_pin_fails([TA.test_clip_inactive_and_skipped_grads])


def test_view_mutant_is_caught(monkeypatch):
    def col_major(stored, view=None, split=None):
        views.validate_view(stored, view, split)
        if view is None:
            return [(0, stored[0], stored[1])]
        r = view[-2]
        n = stored[0] // r
        # wrong: interleaved leading index
        out = []
        for b in range(n):
            off = (b % 2) * (stored[0] // 2) + (b // 2) * r if n % 2 == 0 else b * r
            for q in (split or [r]):
                out.append((off, q, stored[1]))
                off += q
        return out
    monkeypatch.setattr(views, "expand", col_major)
    cases = TV._load("view_examples.json")["cases"]
    assert _some_pin_fails([lambda: [TV.test_view_expansion_matches_bruteforce_reshape(c)
                                     for c in cases]])


@pytest.mark.parametrize("kind", ["wrong_piece_index", "excluded_dropped"])
def test_exclude_mutants_are_caught(monkeypatch, kind):
    import test_oracle_hybrid as TH
    from oracle import hybrid

    def pieces(stored, view=None, split=None, exclude=None):
        ex = set(exclude or ())
        n = len(split) if split is not None else 1
        sl = views.expand(stored, view, split)
        if kind == "wrong_piece_index":     # piece of slice k taken as k // n
            return ([x for k, x in enumerate(sl) if k // n not in ex],
                    [x for k, x in enumerate(sl) if k // n in ex])
        return [x for k, x in enumerate(sl) if k % n not in ex], []   # never sent to AdamW

    monkeypatch.setattr(hybrid, "expand_pieces", pieces)
    with pytest.raises(AssertionError):
        TH.test_excluded_pieces_equal_separate_weights()


@pytest.mark.parametrize("kind", ["linear_cooldown", "floor_relative"])
def test_schedule_mutants_are_caught(monkeypatch, kind):
    import test_oracle_schedule as TS
    from oracle import schedule

    def lr(tokens, peak, warmup=2e9, stable_end=164e9, end=193e9, floor=1e-5):
        if tokens < warmup:
            return peak * tokens / warmup
        if tokens < stable_end:
            return peak
        if tokens < end:
            x = (tokens - stable_end) / (end - stable_end)
            if kind == "linear_cooldown":
                return floor + (peak - floor) * (1.0 - x)
            return peak * (floor + (1 - floor) * (1.0 - math.sqrt(x)))
        return floor if kind == "linear_cooldown" else peak * floor

    monkeypatch.setattr(schedule, "lr_at", lr)
    monkeypatch.setattr(TS, "lr_at", lr)      # the pins bound the name at import
    with pytest.raises(AssertionError):
        for peak in (0.01, 3e-4):
            TS.test_phase_boundaries_from_the_page(peak)
            TS.test_square_root_cooldown_shape(peak)
