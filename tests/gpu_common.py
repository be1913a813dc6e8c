"""Shared helpers of the GPU parity tests (storage <-> device, tolerances).

Tolerances (the arithmetic behind each is in the design notes):
* Newton-Schulz, bf16 path: max-abs <= 2e-2 per slice, and relative
  Frobenius error <= 1.5e-2 (about four bf16 unit roundoffs; the output is
  rounded to bf16 once more after the last product).
* Newton-Schulz, fp32 path: max-abs <= 1e-4.
* fp32 momentum / AdamW moments and updates: normwise relative <= 1e-6,
  ||x - x_ref||_inf <= 1e-6 ||x_ref||_inf.
* Values stored in bf16: equal to the oracle rounded to bf16, with one bf16
  ulp allowed (the GPU rounds an fp32 value that differs from the fp64 one in
  the last fp32 bits, which can cross a bf16 rounding boundary).
"""

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import bf16 as obf16
from oracle.routing import descs_from_specs

NS_BF16_MAXABS = 2e-2
NS_BF16_RELFRO = 1.5e-2
NS_F32_MAXABS = 1e-4
REL_F32 = 1e-6


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible HIP device")


def to_dev(arr: np.ndarray, dtype: str) -> torch.Tensor:
    a = np.ascontiguousarray(arr)
    if dtype == "f32":
        return torch.from_numpy(a.astype(np.float32)).cuda()
    return torch.from_numpy(a.astype(np.uint16).view(np.int16)).view(torch.bfloat16).cuda()


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a device tensor (bf16 / fp32 widen exactly)."""
    if t.dtype == torch.float64:
        return t.detach().cpu().numpy()
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_inf(got: np.ndarray, ref: np.ndarray) -> float:
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / den) if den > 0 else float(np.max(np.abs(got)))


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    m, e = np.frexp(np.abs(x))
    return np.ldexp(np.ones_like(x), np.maximum(e, -125) - 8)


def assert_bf16_close(got: np.ndarray, ref64: np.ndarray, extra: float = 0.0):
    """got (bf16 values) == RNE(ref) within one ulp (plus `extra` absolute)."""
    want = obf16.round_bf16(ref64)
    tol = bf16_ulp(want) + extra
    bad = np.abs(got - want) > tol
    assert not bad.any(), (f"{bad.sum()} of {bad.size} bf16 values off by more than one ulp; "
                           f"max diff {np.max(np.abs(got - want))}")


def assert_ns_close(got: np.ndarray, ref: np.ndarray, precision: str,
                    relfro: float = NS_BF16_RELFRO):
    err = np.max(np.abs(got - ref)) if ref.size else 0.0
    if precision == "bf16":
        assert err <= NS_BF16_MAXABS, f"max-abs {err:.3e}"
        nr = np.linalg.norm(ref)
        if nr > 0:
            rf = np.linalg.norm(got - ref) / nr
            assert rf <= relfro, f"relative Frobenius {rf:.3e}"
        else:
            assert np.all(got == 0)
    else:
        assert err <= NS_F32_MAXABS, f"max-abs {err:.3e}"


def storage_draw(seed: int, step: int, idx: int, shape, std: float, dtype: str) -> np.ndarray:
    return wl.to_storage(wl.draw_f32(seed, step, idx, shape, std), dtype)


TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def build_entries(w: wl.Workload, normuon: bool, init=None):
    """Plan entries (api.Plan) for a workload: device W from the seeded init
    (or ``init``), zero grads and zero optimizer states."""
    from adamw_optimizer_step_amd import _lib as L
    from adamw_optimizer_step_amd import api
    entries = []
    routes, _ = api.route([api.make_desc(p.name, p.shape, p.role, p.no_decay,
                                         p.requires_grad, i, p.view, p.split,
                                         p.exclude)
                           for i, p in enumerate(w.params)])
    for i, (p, r) in enumerate(zip(w.params, routes)):
        W0 = wl.init_weight(w, i) if init is None else init[i]
        e = {"desc": api.make_desc(p.name, p.shape, p.role, p.no_decay, p.requires_grad, i,
                                   p.view, p.split, p.exclude),
             "param": to_dev(W0, p.dtype),
             "grad": torch.zeros(p.shape, dtype=TORCH_DT[p.dtype], device="cuda"),
             "route": r}
        if r[0] == L.MO_ALG_MUON:
            e["momentum"] = torch.zeros(p.shape, dtype=torch.float32, device="cuda")
            if normuon:
                e["normuon_v"] = torch.zeros(p.shape[0], dtype=torch.float32, device="cuda")
        if r[0] == L.MO_ALG_ADAMW or (r[0] == L.MO_ALG_MUON and p.exclude):
            e["exp_avg"] = torch.zeros(p.shape, dtype=torch.float32, device="cuda")
            e["exp_avg_sq"] = torch.zeros(p.shape, dtype=torch.float32, device="cuda")
        entries.append(e)
    return entries


def oracle_descs(w: wl.Workload):
    """Routing descriptors of a workload for oracle.hybrid, with dtypes."""
    descs = descs_from_specs(w.params)
    for d, p in zip(descs, w.params):
        d["dtype"] = p.dtype
    return descs


def relfro(got: np.ndarray, ref: np.ndarray) -> float:
    nr = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / nr) if nr > 0 else float(np.linalg.norm(got))
