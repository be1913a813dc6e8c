"""Python face of the C ABI: torch tensors in, device pointers out.

Argument marshalling only - every step of the optimizer runs in the HIP
library.  Tensors must live on the current HIP device; work is enqueued on
the current torch stream (or the one given) and nothing is synchronised.
Workspaces are torch allocations on the same stream.
"""

from __future__ import annotations

import ctypes as C
from typing import Iterable, List, Optional, Sequence, Tuple

import torch

from . import _lib as L

_DTYPES = {torch.float32: L.MO_F32, torch.bfloat16: L.MO_BF16}


def _dt(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)") from None


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> C.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _dense(t: torch.Tensor, name: str) -> None:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _matrix(t: torch.Tensor, name: str) -> int:
    """Row stride of a row-major 2-D (possibly row-sliced) tensor."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")
    return t.stride(0)


# ---------------------------------------------------------------------------
def muon_momentum(grads: Sequence[Optional[torch.Tensor]], momenta: Sequence[torch.Tensor],
                  dirs: Optional[Sequence[Optional[torch.Tensor]]] = None, mu: float = 0.95,
                  nesterov: bool = True, stream=None) -> None:
    """B <- mu B + G; D <- G + mu B (or B).  A None gradient skips its item."""
    n = len(momenta)
    dirs = list(dirs) if dirs is not None else [None] * n
    items = (L.MomentumItem * max(n, 1))()
    dev = None
    for i, (g, b, d) in enumerate(zip(grads, momenta, dirs)):
        if b.dtype != torch.float32:
            raise TypeError("momentum buffers are fp32")
        _dense(b, "momentum")
        items[i].momentum = _ptr(b)
        items[i].numel = b.numel()
        if g is not None:
            _dense(g, "grad")
            items[i].grad = _ptr(g)
            items[i].grad_dtype = _dt(g)
        if d is not None:
            _dense(d, "dir")
            items[i].dir = _ptr(d)
            items[i].dir_dtype = _dt(d)
        dev = b.device
    if n == 0:
        return
    ws = _workspace(L.lib().muon_momentum_workspace_bytes(n), dev)
    L.check("muon_momentum", L.lib().muon_momentum(items, n, mu, int(bool(nesterov)),
                                                   C.c_void_p(ws.data_ptr()), ws.numel(),
                                                   _stream(stream)))


def _coeff_array(coeffs) -> Tuple[C.Array, int]:
    rows = [tuple(float(x) for x in r) for r in coeffs]
    flat = (C.c_float * (3 * len(rows)))(*[x for r in rows for x in r])
    return flat, len(rows)


PRECISIONS = {"bf16": L.MO_NS_BF16, "fp32": L.MO_NS_F32}


def ns_items(inputs: Sequence[torch.Tensor], outputs: Sequence[torch.Tensor]):
    n = len(inputs)
    items = (L.NsItem * max(n, 1))()
    for i, (x, y) in enumerate(zip(inputs, outputs)):
        if x.shape != y.shape:
            raise ValueError("input / output shape mismatch")
        items[i].inp = _ptr(x)
        items[i].out = _ptr(y)
        items[i].rows, items[i].cols = x.shape
        items[i].ld_in = _matrix(x, "input")
        items[i].ld_out = _matrix(y, "output")
        items[i].in_dtype = _dt(x)
        items[i].out_dtype = _dt(y)
    return items


def ns_options(gram_space: bool = True, big_tile_min_work: Optional[int] = None,
               few_tile_max: Optional[int] = None) -> L.NsOptions:
    """Newton-Schulz options (mo_ns_options); None keeps the library default."""
    o = L.NsOptions()
    L.lib().mo_ns_options_default(C.byref(o))
    o.gram_space = int(bool(gram_space))
    if big_tile_min_work is not None:
        o.big_tile_min_work = int(big_tile_min_work)
    if few_tile_max is not None:
        o.few_tile_max = int(few_tile_max)
    return o


def _ns_opts(options) -> Optional[L.NsOptions]:
    if options is None or isinstance(options, L.NsOptions):
        return options
    return ns_options(**options)


def ns_workspace_bytes(inputs: Sequence[torch.Tensor], precision: str = "bf16", coeffs=None,
                       options=None) -> int:
    """Workspace of ns_orthogonalize_batched; without ``coeffs`` the most any
    coefficient table can need."""
    items = ns_items(inputs, inputs)
    opts = _ns_opts(options)
    flat, steps = _coeff_array(coeffs) if coeffs is not None else (None, 0)
    return int(L.lib().ns_workspace_bytes(items, len(inputs), flat, steps, PRECISIONS[precision],
                                          None if opts is None else C.byref(opts)))


def ns_orthogonalize_batched(inputs: Sequence[torch.Tensor],
                             outputs: Optional[Sequence[torch.Tensor]] = None,
                             coeffs=((1.5, -0.5, 0.0),) * 5, precision: str = "bf16",
                             stream=None, workspace: Optional[torch.Tensor] = None,
                             options=None):
    """Newton-Schulz orthogonalisation of independent 2-D matrices.

    Returns ``outputs`` (new tensors shaped and typed like the inputs when
    not given).  ``coeffs`` is a sequence of per-iteration (a, b, c);
    ``options`` an ``ns_options(...)`` result or a dict of its arguments.
    """
    if outputs is None:
        outputs = [torch.empty_like(x) for x in inputs]
    n = len(inputs)
    items = ns_items(inputs, outputs)
    flat, steps = _coeff_array(coeffs)
    prec = PRECISIONS[precision]
    opts = _ns_opts(options)
    popts = None if opts is None else C.byref(opts)
    need = int(L.lib().ns_workspace_bytes(items, n, flat, steps, prec, popts))
    if workspace is None or workspace.numel() < need:
        workspace = _workspace(need, inputs[0].device)
    L.check("ns_orthogonalize_batched",
            L.lib().ns_orthogonalize_batched(items, n, flat, steps, prec, popts,
                                             C.c_void_p(workspace.data_ptr()),
                                             workspace.numel(), _stream(stream)))
    return outputs


def muon_spectral_estimate(mats: Sequence[torch.Tensor], iters: int = 8,
                           stream=None) -> torch.Tensor:
    """Power-iteration estimate of each fp32 matrix's largest singular value
    (the spectral-cap guard's estimate); returns a float64 device tensor."""
    n = len(mats)
    items = (L.SpectralItem * max(n, 1))()
    for i, m in enumerate(mats):
        if m.dtype != torch.float32:
            raise TypeError("the guard's matrices are fp32 buffers")
        items[i].b = _ptr(m)
        items[i].rows, items[i].cols = m.shape
        items[i].ld = _matrix(m, "matrix")
    out = torch.empty(max(n, 1), dtype=torch.float64, device=mats[0].device)
    ws = _workspace(L.lib().muon_spectral_workspace_bytes(items, n), mats[0].device)
    L.check("muon_spectral_estimate",
            L.lib().muon_spectral_estimate(items, n, int(iters), _ptr(out),
                                           C.c_void_p(ws.data_ptr()), ws.numel(),
                                           _stream(stream)))
    return out[:n]


def normuon_rownorm(O: torch.Tensor, v: torch.Tensor, beta2: float = 0.95, eps: float = 1e-8,
                    stream=None) -> None:
    if v.dtype != torch.float32 or v.numel() != O.shape[0]:
        raise ValueError("v must be fp32 with one entry per row")
    ld = _matrix(O, "O")
    L.check("normuon_rownorm",
            L.lib().normuon_rownorm(_ptr(O), _dt(O), O.shape[0], O.shape[1], ld, _ptr(v), beta2,
                                    eps, _stream(stream)))


def muon_update(W: torch.Tensor, U: torch.Tensor, lr: float, wd: float = 0.0,
                scale: float = 1.0, stream=None) -> None:
    if W.shape != U.shape:
        raise ValueError("W / U shape mismatch")
    L.check("muon_update",
            L.lib().muon_update(_ptr(W), _dt(W), _ptr(U), _dt(U), W.shape[0], W.shape[1],
                                _matrix(W, "W"), _matrix(U, "U"), lr, wd, scale,
                                _stream(stream)))


def _adamw_items(params, grads, exp_avgs, exp_avg_sqs, steps, weight_decay, norm_out):
    n = len(params)
    wds = list(weight_decay) if isinstance(weight_decay, (list, tuple)) else [weight_decay] * n
    items = (L.AdamwItem * max(n, 1))()
    for i in range(n):
        p, g, m, v = params[i], grads[i], exp_avgs[i], exp_avg_sqs[i]
        for t, nm in ((p, "param"), (m, "exp_avg"), (v, "exp_avg_sq")):
            _dense(t, nm)
        if m.dtype != torch.float32 or v.dtype != torch.float32:
            raise TypeError("AdamW moments are fp32")
        if m.numel() != p.numel() or v.numel() != p.numel():
            raise ValueError("AdamW moments must match the param's size")
        items[i].param = _ptr(p)
        items[i].exp_avg = _ptr(m)
        items[i].exp_avg_sq = _ptr(v)
        items[i].numel = p.numel()
        items[i].dtype = _dt(p)
        items[i].step = int(steps[i])
        items[i].weight_decay = float(wds[i])
        if g is not None:
            _dense(g, "grad")
            if g.dtype != p.dtype:
                raise TypeError("grad dtype must match the param dtype")
            if g.numel() != p.numel():
                raise ValueError("grad must match the param's size")
            items[i].grad = _ptr(g)
    if norm_out is not None and (norm_out.dtype != torch.float64 or norm_out.numel() < 1):
        raise TypeError("norm_out must be a float64 device tensor")
    return items


def adamw_clip_step(params: Sequence[torch.Tensor], grads: Sequence[Optional[torch.Tensor]],
                    exp_avgs: Sequence[torch.Tensor], exp_avg_sqs: Sequence[torch.Tensor],
                    steps: Sequence[int], lr: float, beta1: float = 0.9, beta2: float = 0.95,
                    eps: float = 1e-8, weight_decay=0.0, max_norm: float = 1.0,
                    norm_out: Optional[torch.Tensor] = None, stream=None) -> None:
    """Joint clipped AdamW step; ``weight_decay`` is a float or one per param."""
    n = len(params)
    items = _adamw_items(params, grads, exp_avgs, exp_avg_sqs, steps, weight_decay, norm_out)
    dev = params[0].device if n else torch.device("cuda")
    ws = _workspace(L.lib().adamw_workspace_bytes(items, n), dev)
    L.check("adamw_clip_step",
            L.lib().adamw_clip_step(items, n, lr, beta1, beta2, eps, max_norm, _ptr(norm_out),
                                    C.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream)))


def adamw_clip_step_noalloc(params: Sequence[torch.Tensor],
                            grads: Sequence[Optional[torch.Tensor]],
                            exp_avgs: Sequence[torch.Tensor], exp_avg_sqs: Sequence[torch.Tensor],
                            steps: Sequence[int], lr: float, beta1: float = 0.9,
                            beta2: float = 0.95, eps: float = 1e-8, weight_decay=0.0,
                            max_norm: float = 1.0, norm_out: Optional[torch.Tensor] = None,
                            stream=None) -> None:
    """adamw_clip_step with the library's fixed device scratch instead of a
    workspace: nothing is allocated (for code that cannot allocate)."""
    items = _adamw_items(params, grads, exp_avgs, exp_avg_sqs, steps, weight_decay, norm_out)
    L.check("adamw_clip_step_noalloc",
            L.lib().adamw_clip_step_noalloc(items, len(params), lr, beta1, beta2, eps, max_norm,
                                            _ptr(norm_out), _stream(stream)))


# ---------------------------------------------------------------------------
# Host-only: routing and view expansion
# ---------------------------------------------------------------------------
def make_desc(name: str, shape: Sequence[int], role: str = "matrix", no_decay: bool = False,
              requires_grad: bool = True, ident: Optional[int] = None,
              view: Optional[Sequence[int]] = None,
              split: Optional[Sequence[int]] = None,
              exclude: Optional[Sequence[int]] = None) -> L.ParamDesc:
    """``exclude``: split positions whose pieces AdamW steps instead of Muon."""
    d = L.ParamDesc()
    d.name = name.encode()
    d.ident = ident if ident is not None else (hash(name) & 0x7FFFFFFFFFFFFFFF)
    if len(shape) > L.MO_MAX_NDIM:
        raise ValueError("too many dims")
    d.ndim = len(shape)
    for i, s in enumerate(shape):
        d.shape[i] = int(s)
    d.role = L.ROLE_CODES[role]
    d.no_decay = int(bool(no_decay))
    d.requires_grad = int(bool(requires_grad))
    if view is not None:
        if len(view) > L.MO_MAX_NDIM:
            raise ValueError("view rank above the ABI maximum")
        d.view_ndim = len(view)
        for i, s in enumerate(view):
            d.view[i] = int(s)
    if split is not None:
        if len(split) > L.MO_MAX_SPLIT:
            raise ValueError("too many split sizes")
        d.nsplit = len(split)
        for i, s in enumerate(split):
            d.split[i] = int(s)
    for j in exclude or ():
        if not 0 <= int(j) < 32:
            raise ValueError("excluded piece out of range")
        d.exclude_mask |= 1 << int(j)
    return d


def route(descs: Sequence[L.ParamDesc]) -> Tuple[List[Tuple[int, int, int, int]], int]:
    n = len(descs)
    arr = (L.ParamDesc * max(n, 1))(*descs)
    out = (L.RouteOut * max(n, 1))()
    ng = C.c_int32(0)
    L.check("mo_route", L.lib().mo_route(arr, n, out, C.byref(ng)))
    return [(o.algorithm, o.decay, o.group, o.nslices) for o in out[:n]], ng.value


def expand_view(rows: int, cols: int, view: Optional[Sequence[int]] = None,
                split: Optional[Sequence[int]] = None) -> List[Tuple[int, int, int]]:
    v = list(view or [])
    s = list(split or [])
    va = (C.c_int64 * max(len(v), 1))(*v)
    sa = (C.c_int64 * max(len(s), 1))(*s)
    cnt = C.c_int32(0)
    st = L.lib().mo_expand_view(rows, cols, len(v), va, len(s), sa, None, 0, C.byref(cnt))
    if st not in (L.MO_OK, L.MO_EINVAL):
        L.check("mo_expand_view", st)
    out = (C.c_int64 * max(3 * cnt.value, 3))()
    L.check("mo_expand_view", L.lib().mo_expand_view(rows, cols, len(v), va, len(s), sa, out,
                                                     cnt.value, C.byref(cnt)))
    return [(out[3 * i], out[3 * i + 1], out[3 * i + 2]) for i in range(cnt.value)]


# ---------------------------------------------------------------------------
# Plan + grouped step
# ---------------------------------------------------------------------------
# ---------------------------------------------------------------------------
# Host-only: token-clock learning-rate schedule
# ---------------------------------------------------------------------------
def lr_at(tokens: float, peak: float, warmup: float = 2e9, stable_end: float = 164e9,
          end: float = 193e9, floor: float = 1e-5) -> float:
    """Learning rate after ``tokens`` tokens: linear warmup, the peak, then a
    square-root cooldown to ``floor`` (mo_lr_at)."""
    sch = L.LrSchedule(peak, warmup, stable_end, end, floor)
    out = C.c_double()
    L.check("mo_lr_at", L.lib().mo_lr_at(C.byref(sch), float(tokens), C.byref(out)))
    return out.value


class TokenClock:
    """One token clock for both optimizers, each at its own peak: ``advance``
    counts an accepted accumulation window and returns (muon_lr, adamw_lr)."""

    def __init__(self, muon_peak: float = 0.01, adamw_peak: float = 3e-4, **phases):
        self.tokens = 0.0
        self.muon_peak, self.adamw_peak, self.phases = muon_peak, adamw_peak, phases

    def advance(self, window_tokens: float) -> Tuple[float, float]:
        if window_tokens < 0:
            raise ValueError("negative window")
        self.tokens += window_tokens
        return (lr_at(self.tokens, self.muon_peak, **self.phases),
                lr_at(self.tokens, self.adamw_peak, **self.phases))


def make_hparams(muon_lr=0.01, muon_wd=0.0, mu=0.95, nesterov=True, coeffs=((1.5, -0.5, 0.0),) * 5,
                 ns_precision="bf16", normuon=False, normuon_beta2=0.95, normuon_eps=1e-8,
                 adamw_lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, adamw_wd=0.0,
                 max_norm=1.0, spectral_cap=0.0, spectral_iters=8) -> L.HParams:
    h = L.HParams()
    h.muon_lr, h.muon_wd, h.mu, h.nesterov = muon_lr, muon_wd, mu, int(bool(nesterov))
    rows = [tuple(r) for r in coeffs]
    if not 1 <= len(rows) <= L.MO_NS_MAX_STEPS:
        raise ValueError("coefficient table must have 1..64 rows")
    h.ns_steps = len(rows)
    for k, (a, b, c) in enumerate(rows):
        h.ns_coeffs[k][0], h.ns_coeffs[k][1], h.ns_coeffs[k][2] = a, b, c
    h.ns_precision = PRECISIONS[ns_precision]
    h.normuon, h.normuon_beta2, h.normuon_eps = int(bool(normuon)), normuon_beta2, normuon_eps
    h.adamw_lr, h.beta1, h.beta2, h.eps = adamw_lr, beta1, beta2, eps
    h.adamw_wd, h.max_norm = adamw_wd, max_norm
    h.spectral_cap, h.spectral_iters = spectral_cap, int(spectral_iters)
    return h


def plan_options(keep_ns_output: bool = False, **ns) -> L.PlanOptions:
    """Plan options (mo_plan_options): ``keep_ns_output`` and the
    Newton-Schulz options of ``ns_options`` as keyword arguments."""
    o = L.PlanOptions()
    L.lib().mo_plan_options_default(C.byref(o))
    o.ns = ns_options(**ns)
    o.keep_ns_output = int(bool(keep_ns_output))
    return o


def _numel(shape) -> int:
    n = 1
    for d in shape:
        n *= int(d)
    return n


def _check_entry(i: int, e: dict) -> None:
    """Shape, dtype, layout and device of one plan entry's tensors, checked
    before the library records their addresses (it reads G with W's dtype
    and every buffer with W's element count)."""
    d = e["desc"]
    shape = tuple(d.shape[k] for k in range(d.ndim))
    numel = _numel(shape)
    p = e.get("param")
    if p is None:
        return
    if p.numel() != numel:
        raise ValueError(f"entry {i}: param has {p.numel()} elements, descriptor {shape}")
    dev = p.device
    want = {"param": (p.dtype, numel), "grad": (p.dtype, numel),
            "momentum": (torch.float32, numel), "exp_avg": (torch.float32, numel),
            "exp_avg_sq": (torch.float32, numel),
            "normuon_v": (torch.float32, shape[0] if shape else 0)}
    for k, (dt, n) in want.items():
        t = e.get(k)
        if t is None:
            continue
        if t.device != dev:
            raise ValueError(f"entry {i}: {k} on {t.device}, param on {dev}")
        if t.dtype != dt:
            raise TypeError(f"entry {i}: {k} is {t.dtype}, expected {dt}")
        if not t.is_contiguous():
            raise ValueError(f"entry {i}: {k} must be contiguous")
        if t.numel() != n:
            raise ValueError(f"entry {i}: {k} has {t.numel()} elements, expected {n}")


class Plan:
    """Owns a C plan over a parameter table; ``step()`` runs one hybrid step.

    ``entries``: dicts with ``desc`` (a ParamDesc from ``make_desc``), ``param``,
    ``grad`` (or None) and the states the routing needs: ``momentum`` (and
    ``normuon_v`` with NorMuon) for Muon params, ``exp_avg`` / ``exp_avg_sq``
    for AdamW params and for Muon params with excluded pieces (all of the
    param's size).  The tensors must stay alive and in place.  ``options``:
    a ``plan_options(...)`` result or a dict of its arguments.
    """

    def __init__(self, entries: Sequence[dict], hparams: L.HParams, options=None):
        self._setup(entries, options)
        arr = self._param_array(self._keep)
        h = C.c_void_p()
        L.check("mo_plan_create",
                L.lib().mo_plan_create(arr, len(self._keep), C.byref(hparams),
                                       None if self._opts is None else C.byref(self._opts),
                                       C.byref(h)))
        self._h = h

    @classmethod
    def from_groups(cls, groups: Sequence[dict], options=None) -> "Plan":
        """Plan over a group table (mo_plan_create_groups).  ``groups``: dicts
        with ``algorithm`` ('muon' or 'adamw'), ``entries`` (as for the
        constructor) and ``hparams`` (``make_hparams(...)``: the group's own
        learning rate, decay and, for Muon, momentum, coefficient table and
        NorMuon setting).  Plan order is group by group."""
        self = cls.__new__(cls)
        self._setup([e for g in groups for e in g["entries"]], options)
        garr = (L.Group * max(len(groups), 1))()
        self._arrays = []
        for gi, g in enumerate(groups):
            arr = self._param_array(g["entries"])
            self._arrays.append(arr)
            garr[gi].algorithm = {"muon": L.MO_ALG_MUON, "adamw": L.MO_ALG_ADAMW}[g["algorithm"]]
            garr[gi].nparams = len(g["entries"])
            garr[gi].params = C.cast(arr, C.POINTER(L.Param))
            garr[gi].hp = g["hparams"]
        h = C.c_void_p()
        L.check("mo_plan_create_groups",
                L.lib().mo_plan_create_groups(garr, len(groups),
                                              None if self._opts is None else
                                              C.byref(self._opts), C.byref(h)))
        self._h = h
        return self

    def _setup(self, entries, options) -> None:
        self._keep = list(entries)
        if options is not None and not isinstance(options, L.PlanOptions):
            options = plan_options(**options)
        self._opts = options
        # kept on the instance: __del__ may run after module globals are gone
        self._destroy = L.lib().mo_plan_destroy
        self.n = len(self._keep)
        self._ws: Optional[torch.Tensor] = None
        self._slices = None

    @staticmethod
    def _param_array(entries):
        arr = (L.Param * max(len(entries), 1))()
        for i, e in enumerate(entries):
            _check_entry(i, e)
            arr[i].desc = e["desc"]
            arr[i].param = _ptr(e.get("param"))
            arr[i].grad = _ptr(e.get("grad"))
            if e.get("param") is not None:
                arr[i].dtype = _dt(e["param"])
            for k in ("momentum", "normuon_v", "exp_avg", "exp_avg_sq"):
                setattr(arr[i], k, _ptr(e.get(k)))
        return arr

    @property
    def num_groups(self) -> int:
        return int(L.lib().mo_plan_num_groups(self._h))

    def __del__(self):
        h = getattr(self, "_h", None)
        destroy = getattr(self, "_destroy", None)
        if h is not None and h.value and destroy is not None:
            try:
                destroy(h)
            except Exception:  # interpreter teardown
                pass
            self._h = None

    @property
    def workspace_bytes(self) -> int:
        return int(L.lib().mo_plan_workspace_bytes(self._h))

    def routes(self):
        out = (L.RouteOut * max(self.n, 1))()
        L.check("mo_plan_route", L.lib().mo_plan_route(self._h, out, self.n))
        return [(o.algorithm, o.decay, o.group, o.nslices) for o in out[:self.n]]

    def slices(self):
        """(param index, row offset, rows, cols) per Muon slice (fixed at creation)."""
        if self._slices is None:
            k = L.lib().mo_plan_num_slices(self._h)
            out = (C.c_int64 * max(4 * k, 4))()
            L.check("mo_plan_slices", L.lib().mo_plan_slices(self._h, out, k))
            self._slices = [tuple(out[4 * i:4 * i + 4]) for i in range(k)]
        return list(self._slices)

    def get_steps(self) -> List[int]:
        out = (C.c_int32 * max(self.n, 1))()
        L.check("mo_plan_get_steps", L.lib().mo_plan_get_steps(self._h, out, self.n))
        return list(out[:self.n])

    def set_steps(self, steps: Sequence[int]) -> None:
        arr = (C.c_int32 * max(self.n, 1))(*[int(s) for s in steps])
        L.check("mo_plan_set_steps", L.lib().mo_plan_set_steps(self._h, arr, self.n))

    def keep_ns_output(self, keep: bool = True) -> None:
        """Keep each step's Newton-Schulz output O in the workspace (for
        ns_output) instead of applying the update inside the last Newton-Schulz
        launch; the weights are the same bits either way."""
        L.check("mo_plan_keep_ns_output", L.lib().mo_plan_keep_ns_output(self._h, int(bool(keep))))

    def fuses_update(self) -> bool:
        """True if the next step applies the update inside the last
        Newton-Schulz launch."""
        return bool(L.lib().mo_plan_fuses_update(self._h))

    def gram_space(self) -> bool:
        """True if the GEMM-path slices run the Gram-space sequence."""
        return bool(L.lib().mo_plan_gram_space(self._h))

    def slice_algorithms(self) -> List[Tuple[bool, str]]:
        """Per slice of ``slices()``: (Gram space, kernel) with kernel one of
        'gemm128', 'gemm256', 'resident'; None for a slice without gradient."""
        k = len(self.slices())
        out = (C.c_int32 * max(k, 1))()
        L.check("mo_plan_slice_algorithms", L.lib().mo_plan_slice_algorithms(self._h, out, k))
        names = ("gemm128", "gemm256", "resident")
        return [None if v < 0 else (bool(v & 1), names[v >> 1]) for v in out[:k]]

    def ns_output(self, slice_index: int, workspace: Optional[torch.Tensor] = None
                  ) -> torch.Tensor:
        """View into the workspace of one slice's Newton-Schulz output O after
        the last step: (rows, cols) in the stored orientation, bf16 or fp32."""
        ws = self._ws if workspace is None else workspace
        if ws is None:
            raise ValueError("ns_output: the plan has no workspace yet")
        o, ld, dt = C.c_void_p(), C.c_int64(), C.c_int32()
        L.check("mo_plan_ns_output",
                L.lib().mo_plan_ns_output(self._h, int(slice_index), C.c_void_p(ws.data_ptr()),
                                          C.byref(o), C.byref(ld), C.byref(dt)))
        _, _, rows, cols = self._slices[slice_index] if self._slices else \
            self.slices()[slice_index]
        esz = 4 if dt.value == L.MO_F32 else 2
        off = o.value - ws.data_ptr()
        flat = ws[off:off + ((rows - 1) * ld.value + cols) * esz]
        flat = flat.view(torch.float32 if esz == 4 else torch.bfloat16)
        return flat.as_strided((rows, cols), (ld.value, 1))

    def workspace(self, device) -> torch.Tensor:
        if self._ws is None or self._ws.numel() < self.workspace_bytes:
            self._ws = _workspace(self.workspace_bytes, device)
        return self._ws

    def step(self, muon_lr: Optional[float] = None, adamw_lr: Optional[float] = None,
             norm_out: Optional[torch.Tensor] = None, stream=None,
             workspace: Optional[torch.Tensor] = None,
             group_lr: Optional[Sequence[Optional[float]]] = None) -> None:
        """One hybrid step.  ``muon_lr`` / ``adamw_lr`` set every Muon / AdamW
        group's rate this step; ``group_lr[g]`` (None = keep) sets group g's,
        with precedence."""
        a = L.StepArgs()
        a.muon_lr = -1.0 if muon_lr is None else float(muon_lr)
        a.adamw_lr = -1.0 if adamw_lr is None else float(adamw_lr)
        a.norm_out = _ptr(norm_out)
        if group_lr is not None:
            vals = (C.c_float * max(len(group_lr), 1))(
                *[-1.0 if v is None else float(v) for v in group_lr])
            a.group_lr = C.cast(vals, C.POINTER(C.c_float))
            a.n_group_lr = len(group_lr)
        if workspace is None:
            dev = next(e["param"].device for e in self._keep if e.get("param") is not None)
            workspace = self.workspace(dev)
        L.check("mo_grouped_step",
                L.lib().mo_grouped_step(self._h, C.byref(a), C.c_void_p(workspace.data_ptr()),
                                        workspace.numel(), _stream(stream)))
