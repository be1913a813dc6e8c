"""Pins for the token-clock schedule (OMN "Dual-Manifold Optimization" page:
2B-token warmup, peak to 164B, square-root cooldown to a 1e-5 floor at about
193B, separate Muon / AdamW peaks of 0.01 / 3e-4 on one clock)."""

import math

import pytest

from oracle.schedule import TokenClock, lr_at


@pytest.mark.parametrize("peak", [0.01, 3e-4])
def test_phase_boundaries_from_the_page(peak):
    assert lr_at(0.0, peak) == 0.0
    assert lr_at(1e9, peak) == pytest.approx(peak / 2, rel=1e-15)   # halfway through warmup
    assert lr_at(2e9, peak) == peak
    assert lr_at(100e9, peak) == peak
    assert lr_at(164e9, peak) == peak                                 # cooldown starts at peak
    assert lr_at(193e9, peak) == 1e-5
    assert lr_at(500e9, peak) == 1e-5


@pytest.mark.parametrize("peak", [0.01, 3e-4])
def test_square_root_cooldown_shape(peak):
    # a quarter of the way through a square-root cooldown, half of the drop
    # above the floor is gone; a linear one would have lost a quarter
    S, E = 164e9, 193e9
    q = S + (E - S) / 4
    assert lr_at(q, peak) == pytest.approx(1e-5 + (peak - 1e-5) * 0.5, rel=1e-12)
    ninth = S + (E - S) / 9
    assert lr_at(ninth, peak) == pytest.approx(1e-5 + (peak - 1e-5) * (2 / 3), rel=1e-12)
    # continuous at both ends of the cooldown, non-increasing inside it
    eps = 1.0
    # (the square root leaves S with infinite slope: one token drops ~6e-6)
    assert abs(lr_at(S - eps, peak) - lr_at(S + eps, peak)) < 1e-5 * peak
    assert abs(lr_at(E - eps, peak) - lr_at(E, peak)) < 1e-3 * peak
    xs = [S + (E - S) * k / 64 for k in range(65)]
    ys = [lr_at(x, peak) for x in xs]
    assert all(a >= b for a, b in zip(ys, ys[1:]))


def test_one_clock_two_peaks():
    c = TokenClock()
    seen = []
    for w in [0.5e9] * 4 + [80e9, 82e9, 14.5e9, 14.5e9]:
        seen.append(c.advance(w))
    # the ratio of the two rates is the ratio of the peaks until the floor
    # enters (the cooldown mixes in the shared absolute floor)
    for m, a in seen[:6]:
        assert m / a == pytest.approx(0.01 / 3e-4, rel=1e-12)
    assert seen[0] == (pytest.approx(0.0025), pytest.approx(0.000075))
    assert seen[3] == (0.01, 3e-4)
    assert seen[-1] == (1e-5, 1e-5)
    assert c.tokens == 193e9


def test_bad_arguments():
    for kw in ({"tokens": -1.0}, {"warmup": 5e9, "stable_end": 4e9}, {"floor": 1.0}):
        args = dict(tokens=1.0, peak=0.01)
        args.update(kw)
        with pytest.raises(ValueError):
            lr_at(**args)
    assert lr_at(0.0, 0.01, warmup=0.0) == 0.01        # no warmup: peak at once
    assert lr_at(5.0, 0.01, warmup=0.0, stable_end=5.0, end=5.0) == 1e-5
    assert math.isclose(lr_at(3.0, 0.01, warmup=4.0, stable_end=4.0, end=4.0), 0.0075)
