"""One full hybrid Muon + AdamW step over a parameter table, in float64.

Routing follows ``routing.build_groups``; each Muon weight is expanded into
independent slices by ``views.expand``; all AdamW parameters with a gradient
share one clip factor (OMN "Dual-Manifold Optimization" page, recipe
paragraph).  Weights are rounded to their storage dtype after the update.

Excluded split pieces of a Muon weight (Qwen3.8 notes, section 4) are AdamW
parameters of their own: they join the AdamW clip norm and take the AdamW
update with the weight's step counter, and Muon leaves their rows alone
(momentum rows unchanged, no decay, no update).  The notes say only that
these sub-blocks go to AdamW and that the result is gathered back into the
fused layout; the rest is this library's plain reading.
"""

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

from . import adamw as _adamw
from . import bf16 as _bf16
from . import muon as _muon
from .routing import build_groups
from .views import expand_pieces


@dataclass
class HyperParams:
    muon_lr: float = 0.01
    muon_wd: float = 0.0
    mu: float = 0.95
    nesterov: bool = True
    coeffs: np.ndarray = field(default_factory=lambda: np.tile([1.5, -0.5, 0.0], (5, 1)))
    normuon: bool = False
    normuon_beta2: float = 0.95
    normuon_eps: float = 1e-8
    spectral_cap: float = 0.0        # inactive by default (OMN page, Muon-path paragraph)
    spectral_iters: int = 8
    adamw_lr: float = 3e-4
    beta1: float = 0.90
    beta2: float = 0.95
    eps: float = 1e-8
    adamw_wd: float = 0.0
    max_norm: float = 1.0


class HybridState:
    """fp64 optimizer state keyed by parameter name."""

    def __init__(self):
        self.B: Dict[str, np.ndarray] = {}
        self.nv: Dict[str, np.ndarray] = {}
        self.m: Dict[str, np.ndarray] = {}
        self.v: Dict[str, np.ndarray] = {}
        self.t: Dict[str, int] = {}


def hybrid_step(descs: List[dict], W: Dict[str, np.ndarray], G: Dict[str, Optional[np.ndarray]],
                state: HybridState, hp: HyperParams, keep_outputs: bool = False):
    """One step.

    descs: routing descriptors (see ``routing.build_groups``) plus ``dtype``.
    W: name -> fp64 weights (already exact values of the stored dtype).
    G: name -> fp64 gradient or None (skipped this step).
    Returns dict with new weights (rounded to dtype), T, kappa, and when
    ``keep_outputs`` the per-weight Muon intermediates.
    """
    groups = build_groups(descs)
    by_name = {d["name"]: d for d in descs}
    newW = dict(W)
    extras = {}
    adam_items = []
    for g in groups:
        for name in g["names"]:
            d = by_name[name]
            grad = G.get(name)
            if grad is None:
                continue
            if g["algorithm"] == "muon":
                B = state.B.get(name)
                if B is None:
                    B = np.zeros(d["shape"], dtype=np.float64)
                nv = None
                if hp.normuon:
                    nv = state.nv.get(name)
                    if nv is None:
                        nv = np.zeros(d["shape"][0], dtype=np.float64)
                muon_sl, excl = expand_pieces(d["shape"], g["view"], g["split"],
                                              g.get("exclude"))
                res = _muon.muon_param_step(
                    W[name], grad, B, muon_sl,
                    hp.coeffs, hp.muon_lr, hp.mu, hp.muon_wd if g["decay"] else 0.0,
                    hp.nesterov,
                    normuon_v=nv, normuon_beta2=hp.normuon_beta2,
                    normuon_eps=hp.normuon_eps, spectral_cap_value=hp.spectral_cap,
                    spectral_iters=hp.spectral_iters)
                Wm, Bm = res["W"], res["B"]
                for off, r, _ in excl:   # rows that Muon does not own
                    Wm[off:off + r] = W[name][off:off + r]
                    Bm[off:off + r] = B[off:off + r]
                    adam_items.append((name, d, grad, g["decay"], (off, r)))
                state.B[name] = Bm
                if hp.normuon:
                    state.nv[name] = res["v"]
                newW[name] = _bf16.round_to(Wm, d["dtype"])
                if keep_outputs:
                    extras[name] = res
            else:
                adam_items.append((name, d, grad, g["decay"], None))
    T, kappa = 0.0, 1.0
    if adam_items:
        # an item is a whole AdamW weight (rows None) or the rows (off, r) of
        # an excluded piece
        items = []
        for name, d, grad, decay, rows in adam_items:
            t = state.t.get(name, 0) + 1
            m = state.m.get(name, np.zeros(d["shape"], dtype=np.float64))
            v = state.v.get(name, np.zeros(d["shape"], dtype=np.float64))
            sel = slice(None) if rows is None else slice(rows[0], rows[0] + rows[1])
            items.append({"W": W[name][sel], "G": grad[sel], "m": m[sel], "v": v[sel], "t": t,
                          "wd": hp.adamw_wd if decay else 0.0})
        out, T, kappa = _adamw.adamw_clip_step(items, hp.adamw_lr, hp.beta1, hp.beta2,
                                               hp.eps, hp.adamw_wd, hp.max_norm)
        done = set()
        for (name, d, grad, decay, rows), it, res in zip(adam_items, items, out):
            Wn, m, v = res
            if rows is None:
                newW[name] = _bf16.round_to(Wn, d["dtype"])
                state.m[name], state.v[name] = m, v
            else:
                sel = slice(rows[0], rows[0] + rows[1])
                newW[name][sel] = _bf16.round_to(Wn, d["dtype"])
                for st in (state.m, state.v):
                    st.setdefault(name, np.zeros(d["shape"], dtype=np.float64))
                state.m[name][sel], state.v[name][sel] = m, v
            done.add((name, it["t"]))
        for name, t in done:
            state.t[name] = t
    return {"W": newW, "T": T, "kappa": kappa, "muon": extras, "groups": groups}
