"""``MuonAdamW``: a thin optimizer object over the grouped-step plan.

It routes parameters (kimi-k3 "build_parameter_groups" predicate, OMN
"Dual-Manifold Optimization" routing paragraph), allocates the optimizer
state (fp32 momentum for Muon, plus the NorMuon row vector when enabled; fp32
m and v for AdamW) and calls ``mo_grouped_step`` once per ``step()``.
Gradients are read from ``param.grad``; the plan records their addresses, so
keep them in place (``zero_grad(set_to_none=False)``) - a moved or new grad
tensor triggers a plan rebuild.
"""

from __future__ import annotations

from typing import Iterable, List, Optional

import torch

from . import _lib as L
from .api import Plan, make_desc, make_hparams


class MuonAdamW:
    def __init__(self, named_params: Iterable, clock=None, **hparams):
        """``named_params``: iterable of dicts with ``name``, ``param`` and optional
        ``role`` ('matrix' | 'embedding' | 'head' | 'norm'), ``no_decay``,
        ``view``, ``split``, ``exclude`` (split positions stepped by AdamW),
        ``ident`` (tied parameters share one).  ``clock``: an optional
        ``api.TokenClock`` that ``step(window_tokens=...)`` advances."""
        self.entries: List[dict] = []
        self.hp = make_hparams(**hparams)
        for k, e in enumerate(named_params):
            p: torch.Tensor = e["param"]
            desc = make_desc(e["name"], tuple(p.shape), e.get("role", "matrix"),
                             e.get("no_decay", False), p.requires_grad,
                             e.get("ident", id(p)), e.get("view"), e.get("split"),
                             e.get("exclude"))
            self.entries.append({"desc": desc, "param": p, "name": e["name"]})
        from .api import route
        routes, _ = route([e["desc"] for e in self.entries])
        for e, (alg, decay, group, nsl) in zip(self.entries, routes):
            p = e["param"]
            e["algorithm"] = alg
            if alg == L.MO_ALG_MUON:
                e["momentum"] = torch.zeros(p.shape, dtype=torch.float32, device=p.device)
                if self.hp.normuon:
                    e["normuon_v"] = torch.zeros(p.shape[0], dtype=torch.float32,
                                                 device=p.device)
            if alg == L.MO_ALG_ADAMW or (alg == L.MO_ALG_MUON and e["desc"].exclude_mask):
                e["exp_avg"] = torch.zeros(p.shape, dtype=torch.float32, device=p.device)
                e["exp_avg_sq"] = torch.zeros(p.shape, dtype=torch.float32, device=p.device)
        self._plan: Optional[Plan] = None
        self._grad_ptrs = None
        self.clock = clock

    def _current_grads(self):
        return [None if e["param"].grad is None else e["param"].grad.data_ptr()
                for e in self.entries]

    def _build(self):
        steps = self._plan.get_steps() if self._plan is not None else None
        for e in self.entries:
            e["grad"] = e["param"].grad
        self._plan = Plan(self.entries, self.hp)
        if steps is not None:
            self._plan.set_steps(steps)
        self._grad_ptrs = self._current_grads()

    @torch.no_grad()
    def step(self, muon_lr: Optional[float] = None, adamw_lr: Optional[float] = None,
             norm_out: Optional[torch.Tensor] = None,
             window_tokens: Optional[float] = None) -> None:
        """With ``window_tokens`` and a ``clock`` (an ``api.TokenClock``), the
        clock counts the window and sets both rates for this step."""
        if window_tokens is not None:
            if self.clock is None:
                raise ValueError("window_tokens needs a token clock")
            muon_lr, adamw_lr = self.clock.advance(window_tokens)
        if self._plan is None or self._current_grads() != self._grad_ptrs:
            self._build()
        self._plan.step(muon_lr=muon_lr, adamw_lr=adamw_lr, norm_out=norm_out)

    def zero_grad(self) -> None:
        for e in self.entries:
            if e["param"].grad is not None:
                e["param"].grad.zero_()

    def state_dict(self) -> dict:
        st = {}
        for e in self.entries:
            st[e["name"]] = {k: e[k].detach().clone() for k in
                             ("momentum", "normuon_v", "exp_avg", "exp_avg_sq") if k in e}
        st["__steps__"] = self._plan.get_steps() if self._plan is not None else None
        return st

    def load_state_dict(self, st: dict) -> None:
        for e in self.entries:
            for k, v in st.get(e["name"], {}).items():
                e[k].copy_(v)
        if st.get("__steps__") is not None:
            if self._plan is None:
                self._build()
            self._plan.set_steps(st["__steps__"])
