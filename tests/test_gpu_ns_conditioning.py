"""Newton-Schulz parity on badly conditioned inputs, through every Gram-space
route and through the plain iteration.

The NorMuon paper (section 1, Figure 1a) describes momentum matrices with a
few dominant singular directions.  Two seeded stand-ins:
* ``spike``: the N(0, 1e-3) gradient plus a rank-8 component at 100x;
* ``spectrum``: U diag(sigma) V^T with sigma spaced geometrically from 1 down
  to 1e-4.

Gram space carries A = X X^T, whose small eigenvalues are the squares of X's
small singular values; the library admits it only while the table's gain
prod_k a_k^2 is at most 1024 (cubic up to 8 iterations, quintic up to 5).
Each case runs with Gram space allowed (the default) and with the plain
iteration, and meets the bf16 bound max|O - O_ref| <= 2e-2 either way.  The
relative Frobenius error on such inputs grows with the table's gain in both
algorithms (the noise directions are amplified, their rounding is set by the
dominant ones); it is bounded here for the default five cubic iterations,
and the CPU emulation test covers its growth.
"""

import math

import numpy as np
import pytest
import torch

import workloads as wl
from adamw_optimizer_step_amd import api
from oracle import muon as omuon

from gpu_common import (NS_BF16_MAXABS, NS_BF16_RELFRO, build_entries, f64, relfro,
                        require_gpu, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _input(kind: str, index: int, shape):
    r, c = shape
    if kind == "spike":
        w = wl.Workload("spike", 71, (wl.ParamSpec("w", shape, "bf16"),), grad_std=1e-3)
        return wl.spiked_grad(w, 0, 1 + index)
    return wl.prescribed_spectrum(72, index, r, c, 1.0, 1e-4)


TABLES = {"cubic5": (wl.CUBIC, 5), "cubic7": (wl.CUBIC, 7), "quintic5": (wl.QUINTIC, 5),
          "quintic7": (wl.QUINTIC, 7)}


def _gain(table) -> float:
    return math.prod(a * a for a, _, _ in table)


def _check(got: np.ndarray, ref: np.ndarray, table_key: str, what: str) -> None:
    err = float(np.max(np.abs(got - ref)))
    rf = relfro(got, ref)
    print(f"[conditioning] {what}: max-abs {err:.3e} relfro {rf:.3e}", flush=True)
    assert err <= NS_BF16_MAXABS, f"{what}: max-abs {err:.3e}"
    if table_key == "cubic5":
        assert rf <= NS_BF16_RELFRO, f"{what}: relative Frobenius {rf:.3e}"


# GEMM path, rectangular (Gram space for cubic-type tables) on 128 x 128
# tiles; slice-resident, short sides 64 and 128, both orientations
STANDALONE_SHAPES = [(384, 200), (200, 384), (64, 256), (256, 64), (128, 512), (512, 128),
                     (96, 1000)]


@pytest.mark.parametrize("kind", ["spike", "spectrum"])
@pytest.mark.parametrize("table_key", list(TABLES))
@pytest.mark.parametrize("mode", ["gram_space", "plain"])
def test_ill_conditioned_standalone(kind, table_key, mode):
    row, steps = TABLES[table_key]
    cf = [row] * steps
    mats = [_input(kind, i, s) for i, s in enumerate(STANDALONE_SHAPES)]
    outs = api.ns_orthogonalize_batched([to_dev(m, "bf16") for m in mats], coeffs=cf,
                                        options={"gram_space": mode == "gram_space"})
    for shape, m, o in zip(STANDALONE_SHAPES, mats, outs):
        D = wl.from_storage(m, "bf16").astype(np.float64)
        _check(f64(o), omuon.newton_schulz(D, cf), table_key,
               f"{kind} {table_key} {mode} {shape}")


@pytest.mark.parametrize("kind", ["spike", "spectrum"])
@pytest.mark.parametrize("table_key", ["cubic5", "cubic7"])
def test_ill_conditioned_big_tiles(kind, table_key):
    """Rectangular slices on 256 x 256 tiles, in Gram space (cubic rows)."""
    row, steps = TABLES[table_key]
    cf = [row] * steps
    shapes = [(1100, 530), (530, 1100)]
    mats = [_input(kind, 10 + i, s) for i, s in enumerate(shapes)]
    outs = api.ns_orthogonalize_batched([to_dev(m, "bf16") for m in mats], coeffs=cf,
                                        options={"big_tile_min_work": 0})
    for shape, m, o in zip(shapes, mats, outs):
        D = wl.from_storage(m, "bf16").astype(np.float64)
        _check(f64(o), omuon.newton_schulz(D, cf), table_key, f"{kind} {table_key} {shape}")


@pytest.mark.parametrize("table_key", list(TABLES))
def test_gram_space_rule(table_key):
    """The plan runs Gram space exactly when the table's gain allows it."""
    row, steps = TABLES[table_key]
    w = wl.Workload("rule", 73, (wl.ParamSpec("w", (256, 640), "bf16"),
                                 wl.ParamSpec("h", (128, 512), "bf16")))
    plan = api.Plan(build_entries(w, normuon=False), api.make_hparams(coeffs=[row] * steps))
    assert plan.gram_space() == (_gain([row] * steps) <= 1024.0)


@pytest.mark.parametrize("kind", ["spike", "spectrum"])
@pytest.mark.parametrize("mode", ["gram_space", "plain"])
def test_ill_conditioned_grouped_gate_shape(kind, mode):
    """The grouped step at the dense decoder's FFN shapes, gate (5632, 2048)
    and down (2048, 5632), with a badly conditioned gradient: the Newton-Schulz
    output of both slices against the oracle, in Gram space (the default for
    these rectangular slices) and in the plain iteration."""
    shapes = [(5632, 2048), (2048, 5632)]
    w = wl.Workload("gate_shape", 74, tuple(wl.ParamSpec(f"w{i}", s, "bf16")
                                             for i, s in enumerate(shapes)), grad_std=1e-3)
    ents = build_entries(w, normuon=False)
    plan = api.Plan(ents, api.make_hparams(),
                    options={"gram_space": mode == "gram_space", "keep_ns_output": True})
    assert plan.gram_space() == (mode == "gram_space")
    for i, (e, p) in enumerate(zip(ents, w.params)):
        e["grad"].copy_(to_dev(_input(kind, 20 + i, p.shape), "bf16"))
    G = [f64(e["grad"]) for e in ents]
    plan.step()
    torch.cuda.synchronize()
    cf = wl.coeff_table("cubic")
    for k, (param, off, r, c) in enumerate(plan.slices()):
        _, D = omuon.momentum(np.zeros_like(G[param]), G[param], wl.MUON_MU)
        _check(f64(plan.ns_output(k)), omuon.newton_schulz(D[off:off + r], cf), "cubic5",
               f"grouped {kind} {mode} ({r}, {c})")
