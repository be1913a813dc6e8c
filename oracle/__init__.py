"""fp64 CPU oracle for the hybrid Muon + AdamW optimizer step.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow reference that the
HIP library is checked against.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; the product path
never does, and it imports nothing from the product package.

Everything is float64 numpy, written step by step from the pages:

* ``views``   - view / split expansion into independent row slabs
                (kimi-k3 "build_parameter_groups": "Recording independent
                matrix geometry", "The layout declarations are literal").
* ``routing`` - the Muon / AdamW routing predicate and grouping
                (same page: "Exclusion and decay rules", "Classification
                happens once per original parameter identity"; OMN
                "Dual-Manifold Optimization": routing paragraph).
* ``muon``    - momentum, Nesterov direction, max-abs and Frobenius
                normalisation, Newton-Schulz iterations, NorMuon row
                normalisation, shape scale and update (OMN page, Muon-path
                and rectangular-scaling paragraphs; NorMuon paper section 2.2
                eqs. (1)-(5) and section 3.1).
* ``adamw``   - global-norm clip over the AdamW parameters and the AdamW
                update (OMN page, recipe paragraph; Qwen3.8 optimizer notes,
                "Adam/AdamW" background).
* ``hybrid``  - one full hybrid step over a parameter table, with excluded
                pieces of fused weights (Qwen3.8 optimizer notes, section 4).
* ``schedule``- the token-clock learning-rate schedule (OMN page, opening
                summary and the recipe paragraph on separate peaks).
* ``bf16``    - exact widening of bf16 storage and fp64 -> bf16 rounding.

Parity status: every function here is pinned by a ``-m "not gpu"`` test
against values the pages print, closed forms, invariants or brute force
(``tests/test_oracle_*.py``), with one exception: Newton-Schulz outputs for a
*general* matrix after the fixed number of iterations are pinned only through
the prescribed-SVD closed form (exact for every input built that way); no page
prints such values.
"""

from . import adamw, bf16, hybrid, muon, routing, schedule, views  # noqa: F401
