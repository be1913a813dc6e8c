"""Token-clock learning-rate schedule (OMN "Dual-Manifold Optimization" page,
opening summary and the recipe paragraph on separate peaks).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The page fixes the phases by tokens seen: a 2B-token warmup, the peak held
until 164B tokens, then a square-root cooldown to an absolute floor of 1e-5
at roughly 193B tokens; the Muon and AdamW rates follow the same phases, each
from its own peak (0.01 and 3e-4), driven by one token clock that advances
once per accepted accumulation window.  It prints no formula, so the plain
reading is written out here:

* warmup, 0 <= tau < W:        lr = peak * tau / W   (linear from zero);
* stable, W <= tau < S:        lr = peak;
* cooldown, S <= tau < E:      lr = floor + (peak - floor) * (1 - sqrt(x)),
                               x = (tau - S) / (E - S);
* after the end, tau >= E:     lr = floor.

tau is the clock after the current window's tokens are counted, so the first
window already trains at a positive rate.
"""

import math


def lr_at(tokens: float, peak: float, warmup: float = 2e9, stable_end: float = 164e9,
          end: float = 193e9, floor: float = 1e-5) -> float:
    if tokens < 0 or not (0 <= warmup <= stable_end <= end) or not (0 <= floor <= peak):
        raise ValueError("bad schedule arguments")
    if tokens < warmup:
        return peak * tokens / warmup
    if tokens < stable_end:
        return peak
    if tokens < end:
        x = (tokens - stable_end) / (end - stable_end)
        return floor + (peak - floor) * (1.0 - math.sqrt(x))
    return floor


class TokenClock:
    """One clock for both optimizers: ``advance`` counts an accepted window
    and returns the (Muon, AdamW) rates for the step it takes."""

    def __init__(self, muon_peak: float = 0.01, adamw_peak: float = 3e-4, **phases):
        self.tokens = 0.0
        self.muon_peak, self.adamw_peak, self.phases = muon_peak, adamw_peak, phases

    def advance(self, window_tokens: float):
        if window_tokens < 0:
            raise ValueError("negative window")
        self.tokens += window_tokens
        return (lr_at(self.tokens, self.muon_peak, **self.phases),
                lr_at(self.tokens, self.adamw_peak, **self.phases))
