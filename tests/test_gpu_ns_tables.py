"""GPU parity with per-iteration coefficient tables whose rows differ.

The NorMuon paper's eq. (5) takes (a, b, c) per iteration, and the Qwen3.8
optimizer notes (section 2) run eight iterations with a per-step schedule.
Each table here is checked against the oracle through every kernel that
reads the table (the batched GEMM launches, one per phase and iteration; the
slice-resident kernel, which indexes the rows itself; the Gram-space
sequence), through ns_orthogonalize_batched and through mo_grouped_step.

Besides the usual tolerances, every output must lie closer to the oracle's
result for the table than half the distance (relative Frobenius) from that
result to the oracle's result for a mis-indexed reading of the table:
reversed, row 0 only, the next row, the previous row.  That distance is
computed on the same input and asserted to be at least 1e-2, so a kernel that
mis-indexed the rows in any of those ways fails.
"""

import numpy as np
import pytest
import torch

import workloads as wl
from adamw_optimizer_step_amd import api
from oracle import muon as omuon

from gpu_common import (assert_ns_close, build_entries, f64, relfro, require_gpu,
                        storage_draw, to_dev)

pytestmark = pytest.mark.gpu

Q = (15 / 8, -10 / 8, 3 / 8)
# eight cubic-type rows (a, 1 - a, 0) with distinct a; small-singular-value
# gain prod a^2 = 113, so the bf16 path may run them in Gram space
SCHED8 = [(a, 1.0 - a, 0.0) for a in (2.0, 1.0, 1.8, 1.1, 1.6, 1.2, 1.4, 1.0)]
# cubic-type (c = 0) and quintic-type (c != 0) rows mixed, identity rows included
MIXED6 = [(2.0, -1.0, 0.0), (1.0, 0.0, 0.0), Q, (1.3, -0.3, 0.0), Q, (1.0, 0.0, 0.0)]
TABLES = {"sched8": SCHED8, "mixed6": MIXED6}


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _misread(table):
    t = [tuple(r) for r in table]
    return {"reversed": t[::-1], "row0_only": [t[0]] * len(t),
            "next_row": t[1:] + [t[-1]], "previous_row": [t[0]] + t[:-1]}


def _check_table(got: np.ndarray, D: np.ndarray, table, precision: str) -> None:
    ref = omuon.newton_schulz(D, table)
    assert_ns_close(got, ref, precision)
    err = relfro(got, ref)
    for name, t in _misread(table).items():
        gap = relfro(omuon.newton_schulz(D, t), ref)
        assert gap >= 1e-2, f"the table cannot be told from its {name} reading ({gap:.3e})"
        assert err < gap / 2, f"output {err:.3e} from the table, {name} reading at {gap:.3e}"


# GEMM path: rectangular (Gram space for cubic-type tables), square (plain),
# both orientations; slice-resident: short sides 64-128 (Gram space) and 33
# (plain)
STANDALONE_SHAPES = [(300, 200), (200, 384), (256, 256), (64, 256), (96, 1000), (128, 512),
                     (392, 120), (33, 600)]


@pytest.mark.parametrize("table", list(TABLES))
@pytest.mark.parametrize("mode", ["gram_space", "plain", "fp32"])
def test_distinct_rows_standalone(table, mode):
    cf = TABLES[table]
    precision = "fp32" if mode == "fp32" else "bf16"
    dtype = "f32" if mode == "fp32" else "bf16"
    mats = [storage_draw(61, 1, i, s, 1.0, dtype) for i, s in enumerate(STANDALONE_SHAPES)]
    outs = api.ns_orthogonalize_batched([to_dev(m, dtype) for m in mats], coeffs=cf,
                                        precision=precision,
                                        options={"gram_space": mode == "gram_space"})
    for shape, m, o in zip(STANDALONE_SHAPES, mats, outs):
        D = wl.from_storage(m, dtype).astype(np.float64)
        print(f"[tables] {table} {mode} {shape}", flush=True)
        _check_table(f64(o), D, cf, precision)


@pytest.mark.parametrize("table", list(TABLES))
def test_distinct_rows_big_tiles(table):
    """256 x 256 tiles (short sides >= 512) with a distinct-row table."""
    cf = TABLES[table]
    shapes = [(1100, 530), (530, 1100)]
    mats = [storage_draw(62, 1, i, s, 1.0, "bf16") for i, s in enumerate(shapes)]
    outs = api.ns_orthogonalize_batched([to_dev(m, "bf16") for m in mats], coeffs=cf,
                                        options={"big_tile_min_work": 0})
    for m, o in zip(mats, outs):
        D = wl.from_storage(m, "bf16").astype(np.float64)
        _check_table(f64(o), D, cf, "bf16")


def _grouped_shapes():
    ps = [wl.ParamSpec("norm", (64,), "bf16", wl.ROLE_NORM, no_decay=True),
          wl.ParamSpec("square", (256, 256), "bf16"),
          wl.ParamSpec("wide", (256, 640), "bf16"),
          wl.ParamSpec("tall", (512, 256), "bf16"),
          wl.ParamSpec("padded", (200, 336), "bf16"),
          wl.ParamSpec("small_wide", (96, 256), "bf16"),
          wl.ParamSpec("small_tall", (392, 120), "bf16"),
          wl.ParamSpec("heads", (256, 512), "bf16", view=(2, 128, 512)),
          wl.ParamSpec("kv", (80, 64), "bf16", view=(2, 40, 64), split=(16, 24))]
    return wl.Workload("table_shapes", 19, tuple(ps), grad_std=1e-3)


@pytest.mark.parametrize("table", list(TABLES))
@pytest.mark.parametrize("mode", ["gram_space", "plain"])
def test_distinct_rows_grouped(table, mode):
    """The grouped step reads the plan's table: every slice's O (kept in the
    workspace) against the oracle, in Gram space and in the plain iteration;
    iteration 0 reads D in place for the square and wide slices."""
    cf = TABLES[table]
    w = _grouped_shapes()
    ents = build_entries(w, normuon=False)
    plan = api.Plan(ents, api.make_hparams(coeffs=cf),
                    options={"gram_space": mode == "gram_space", "keep_ns_output": True})
    assert plan.gram_space() == (mode == "gram_space")
    for i, (e, p) in enumerate(zip(ents, w.params)):
        e["grad"].copy_(to_dev(wl.grad(w, i, 1), p.dtype))
    G = [f64(e["grad"]) for e in ents]
    plan.step()
    torch.cuda.synchronize()
    for k, (param, off, r, c) in enumerate(plan.slices()):
        _, D = omuon.momentum(np.zeros_like(G[param]), G[param], wl.MUON_MU)
        print(f"[tables] grouped {table} {mode} slice {k} ({r}, {c})", flush=True)
        if min(r, c) >= 64:
            _check_table(f64(plan.ns_output(k)), D[off:off + r], cf, "bf16")
        else:
            assert_ns_close(f64(plan.ns_output(k)), omuon.newton_schulz(D[off:off + r], cf),
                            "bf16")
