"""GPU parity of the grouped hybrid step (mo_grouped_step) against the oracle's
hybrid step, plus the fused-versus-separate gate/up invariant."""

import math

import numpy as np
import pytest
import torch

import workloads as wl
from adamw_optimizer_step_amd import _lib as L
from adamw_optimizer_step_amd import api
from oracle import muon as omuon
from oracle.hybrid import HybridState, HyperParams, hybrid_step
from oracle.views import expand, expand_pieces

from gpu_common import (NS_BF16_MAXABS, NS_F32_MAXABS, REL_F32,
                        assert_bf16_close, assert_ns_close, bf16_ulp, build_entries, f64,
                        oracle_descs, rel_inf, require_gpu, to_dev)

pytestmark = pytest.mark.gpu

@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("precision", ["fp32", "bf16"])
def test_grouped_tiny_three_steps(precision):
    w = wl.tiny_routing()
    ents = build_entries(w, normuon=False)
    coeffs = wl.coeff_table("cubic")
    plan = api.Plan(ents, api.make_hparams(coeffs=coeffs, ns_precision=precision))
    descs = oracle_descs(w)
    st = HybridState()
    hp = HyperParams(coeffs=coeffs)
    Wref = {p.name: f64(e["param"]) for p, e in zip(w.params, ents)}
    norm = torch.zeros(1, dtype=torch.float64, device="cuda")
    tol_ns = NS_F32_MAXABS if precision == "fp32" else NS_BF16_MAXABS
    for step in (1, 2, 3):
        G = {}
        for i, (p, e) in enumerate(zip(w.params, ents)):
            g = wl.grad(w, i, step)
            e["grad"].copy_(to_dev(g, p.dtype))
            G[p.name] = wl.from_storage(g, p.dtype).astype(np.float64)
        Wold = {p.name: f64(e["param"]) for p, e in zip(w.params, ents)}
        plan.step(norm_out=norm)
        out = hybrid_step(descs, Wref, G, st, hp, keep_outputs=True)
        assert abs(f64(norm)[0] - out["T"]) <= 1e-12 * out["T"]
        for p, e in zip(w.params, ents):
            got = f64(e["param"])
            if p.name in out["muon"]:
                res = out["muon"][p.name]
                assert rel_inf(f64(e["momentum"]), res["B"]) <= REL_F32
                dgot, dref = got - Wold[p.name], -0.01 * res["U"]
                for off, r, c in expand(p.shape, p.view, p.split):
                    sc = math.sqrt(max(1.0, r / c))
                    err = np.abs(dgot[off:off + r] - dref[off:off + r]).max()
                    assert err <= 0.01 * sc * tol_ns + 1e-7, (p.name, off, err)
            else:
                dgot, dref = got - Wold[p.name], out["W"][p.name] - Wold[p.name]
                tol = REL_F32 * np.abs(dref).max() + 2 ** -23 * np.abs(got).max()
                assert np.max(np.abs(dgot - dref)) <= tol, p.name
                assert rel_inf(f64(e["exp_avg"]), st.m[p.name]) <= REL_F32
                assert rel_inf(f64(e["exp_avg_sq"]), st.v[p.name]) <= REL_F32
            Wref[p.name] = got.copy()     # continue both sides from the stored weights
    assert plan.get_steps() == [3, 0, 0, 0, 3]


def _small_decoder(fused: bool, normuon: bool, dtype="bf16"):
    d, ffn = 64, 96
    ps = [wl.ParamSpec("embed", (256, d), dtype, wl.ROLE_EMBEDDING, no_decay=True),
          wl.ParamSpec("norm1", (d,), dtype, wl.ROLE_NORM, no_decay=True),
          wl.ParamSpec("q", (d, d), dtype)]
    if fused:
        ps.append(wl.ParamSpec("gate_up", (2 * ffn, d), dtype, view=(2, ffn, d)))
    else:
        ps += [wl.ParamSpec("gate", (ffn, d), dtype), wl.ParamSpec("up", (ffn, d), dtype)]
    ps.append(wl.ParamSpec("down", (d, ffn), dtype))
    return wl.Workload("small_decoder", 7, tuple(ps), grad_std=1e-3, normuon=normuon)


def _run_small(fused, normuon, steps=2, precision="bf16"):
    w = _small_decoder(fused, normuon)
    # identical data for the fused and separate layouts: build the fused
    # weights by stacking the separate ones
    sep = _small_decoder(False, normuon)
    init_sep = [wl.init_weight(sep, i) for i in range(len(sep.params))]
    grads_sep = {t: [wl.grad(sep, i, t) for i in range(len(sep.params))]
                 for t in range(1, steps + 1)}
    def fuse(arrs):
        return arrs[:3] + [np.concatenate([arrs[3], arrs[4]], axis=0), arrs[5]] if fused else arrs
    ents = build_entries(w, normuon, init=fuse(init_sep))
    plan = api.Plan(ents, api.make_hparams(ns_precision=precision, normuon=normuon))
    for t in range(1, steps + 1):
        for e, g, p in zip(ents, fuse(grads_sep[t]), w.params):
            e["grad"].copy_(to_dev(g, p.dtype))
        plan.step()
    return w, ents, init_sep, grads_sep


@pytest.mark.parametrize("normuon", [False, True])
def test_fused_gate_up_equals_separate(normuon):
    _, fused, _, _ = _run_small(True, normuon)
    _, sep, _, _ = _run_small(False, normuon)
    fw = f64(fused[3]["param"])
    assert np.array_equal(fw[:96], f64(sep[3]["param"]))
    assert np.array_equal(fw[96:], f64(sep[4]["param"]))
    if normuon:
        fv = f64(fused[3]["normuon_v"])
        assert np.array_equal(fv[:96], f64(sep[3]["normuon_v"]))
        assert np.array_equal(fv[96:], f64(sep[4]["normuon_v"]))
    for a, b in ((0, 0), (2, 2), (4, 5)):
        assert np.array_equal(f64(fused[a]["param"]), f64(sep[b]["param"]))


@pytest.mark.parametrize("precision", ["bf16", "fp32"])
def test_grouped_normuon_parity(precision):
    """NorMuon in the grouped step (NorMuon paper section 3.1), over two
    steps: each slice's Newton-Schulz output O element-wise against the
    oracle's (1e-4 fp32 path, 2e-2 bf16 path); then, from the GPU's own O,
    the row second moment v (EMA of the row mean square) and the weights
    W (1 - lr wd) - lr scale O / (sqrt(v) + eps).  Momentum and the AdamW
    params against the oracle as usual."""
    w = _small_decoder(False, True)
    ents = build_entries(w, normuon=True)
    plan = api.Plan(ents, api.make_hparams(ns_precision=precision, normuon=True))
    assert not plan.fuses_update()
    descs = oracle_descs(w)
    st = HybridState()
    hp = HyperParams(normuon=True)
    Wref = {p.name: f64(e["param"]) for p, e in zip(w.params, ents)}
    for t in (1, 2):
        G = {}
        for i, (p, e) in enumerate(zip(w.params, ents)):
            g = wl.grad(w, i, t)
            e["grad"].copy_(to_dev(g, p.dtype))
            G[p.name] = wl.from_storage(g, p.dtype).astype(np.float64)
        Wold = {p.name: f64(e["param"]) for p, e in zip(w.params, ents)}
        vold = {p.name: f64(e["normuon_v"]) for p, e in zip(w.params, ents) if "normuon_v" in e}
        plan.step()
        torch.cuda.synchronize()
        out = hybrid_step(descs, Wref, G, st, hp, keep_outputs=True)
        slices = plan.slices()
        for pi, (p, e) in enumerate(zip(w.params, ents)):
            got = f64(e["param"])
            if p.name not in out["muon"]:
                assert_bf16_close(got, out["W"][p.name])
                Wref[p.name] = got.copy()
                continue
            res = out["muon"][p.name]
            assert rel_inf(f64(e["momentum"]), res["B"]) <= REL_F32
            for k, (owner, off, r, c) in enumerate(slices):
                if owner != pi:
                    continue
                rows = slice(off, off + r)
                print(f"[normuon] {precision} step {t} {p.name} rows {off}:{off + r}", flush=True)
                O = f64(plan.ns_output(k))
                assert_ns_close(O, res["O"][rows], precision)
                On, v_exp = omuon.normuon_rownorm(O, vold[p.name][rows], hp.normuon_beta2,
                                                  hp.normuon_eps)
                assert rel_inf(f64(e["normuon_v"])[rows], v_exp) <= 1e-5
                sc = math.sqrt(max(1.0, r / c))
                assert_bf16_close(got[rows], omuon.apply_update(Wold[p.name][rows], sc * On, 0.01),
                                  extra=2e-6 * 0.01 * sc * np.abs(On))
            Wref[p.name] = got.copy()
    assert plan.get_steps() == [2, 2, 0, 0, 0, 0]


def _three_chains():
    """One batch whose Newton-Schulz launches form all three chains: a
    Gram-space GEMM sequence (wide), the plain GEMM iteration (square) and
    the slice-resident kernel (128 rows), beside AdamW params."""
    ps = [wl.ParamSpec("embed", (256, 64), "bf16", wl.ROLE_EMBEDDING, no_decay=True),
          wl.ParamSpec("norm", (64,), "bf16", wl.ROLE_NORM, no_decay=True),
          wl.ParamSpec("square", (384, 384), "bf16"),
          wl.ParamSpec("wide", (256, 640), "bf16"),
          wl.ParamSpec("tall", (520, 200), "bf16"),
          wl.ParamSpec("head", (128, 512), "bf16"),
          wl.ParamSpec("heads", (192, 256), "bf16", view=(3, 64, 256))]
    return wl.Workload("three_chains", 13, tuple(ps), grad_std=1e-3)


def _run_chains(steps=2):
    w = _three_chains()
    ents = build_entries(w, normuon=False)
    plan = api.Plan(ents, api.make_hparams(muon_wd=0.1))
    kinds = {a for a in plan.slice_algorithms() if a is not None}
    assert {(True, "gemm128"), (False, "gemm128"), (True, "resident")} <= kinds, kinds
    for t in range(1, steps + 1):
        for i, (e, p) in enumerate(zip(ents, w.params)):
            e["grad"].copy_(to_dev(wl.grad(w, i, t), p.dtype))
        plan.step()
    return w, ents


@pytest.mark.parametrize("case", ["small_decoder", "three_chains"])
def test_overlapped_step_equals_serial(case):
    """AdamW on one side stream and the batch's independent Newton-Schulz
    chains split over the caller's stream and a second one (the default),
    against every kernel in order on one stream (what the step does while
    kernel timing is on): the same kernels read and write disjoint buffers,
    so the results are bit-identical."""
    run = (lambda: _run_small(False, False)[1]) if case == "small_decoder" else \
        (lambda: _run_chains()[1])
    over = run()
    torch.cuda.synchronize()
    lib = L.lib()
    L.check("timing", lib.mo_timing_enable(1))
    try:
        serial = run()
        torch.cuda.synchronize()
    finally:
        L.check("timing", lib.mo_timing_enable(0))
    for a, b in zip(over, serial):
        for k in ("param", "momentum", "exp_avg", "exp_avg_sq"):
            if k in a:
                assert torch.equal(a[k], b[k]), (a["desc"].name, k)


def _mixed_shapes():
    """Slices for every kernel that can finish a step: slice-resident (wide,
    tall, split view), 128 x 128 GEMM tiles (wide, tall), 256 x 256 tiles
    (with big_tile_min_work = 0), fp32 weights, and AdamW params."""
    ps = [wl.ParamSpec("embed", (256, 64), "bf16", wl.ROLE_EMBEDDING, no_decay=True),
          wl.ParamSpec("norm", (64,), "bf16", wl.ROLE_NORM, no_decay=True),
          wl.ParamSpec("small_wide", (96, 256), "bf16"),
          wl.ParamSpec("small_tall", (392, 120), "bf16"),
          wl.ParamSpec("kv", (80, 64), "bf16", view=(2, 40, 64), split=(16, 24)),
          wl.ParamSpec("gemm_wide", (200, 336), "bf16"),
          wl.ParamSpec("gemm_tall", (344, 192), "bf16"),
          wl.ParamSpec("big", (520, 776), "bf16"),
          wl.ParamSpec("f32_tall", (136, 48), "f32")]
    return wl.Workload("mixed_shapes", 11, tuple(ps), grad_std=1e-3)


@pytest.mark.parametrize("mode", ["gram_space", "plain"])
@pytest.mark.parametrize("big_tiles", [False, True])
def test_fused_update_bit_identical(big_tiles, mode):
    """The Muon update applied inside the last Newton-Schulz launch (the
    default) gives the same bits as the separate row pass over the stored O,
    for every kernel that can end a step, over two steps, in the Gram-space
    sequence and in the plain iteration."""
    opts = {"big_tile_min_work": 0 if big_tiles else None, "gram_space": mode == "gram_space"}
    w = _mixed_shapes()
    runs = []
    for keep in (True, False):
        ents = build_entries(w, normuon=False)
        plan = api.Plan(ents, api.make_hparams(muon_wd=0.1), options=opts)
        plan.keep_ns_output(keep)
        assert plan.fuses_update() == (not keep)
        for t in (1, 2):
            for i, (e, p) in enumerate(zip(ents, w.params)):
                e["grad"].copy_(to_dev(wl.grad(w, i, t), p.dtype))
            plan.step()
        torch.cuda.synchronize()
        runs.append(ents)
    for a, b, p in zip(runs[0], runs[1], w.params):
        for k in ("param", "momentum", "exp_avg", "exp_avg_sq"):
            if k in a:
                assert torch.equal(a[k], b[k]), (p.name, k)
    # the weights did move
    assert not torch.equal(runs[1][5]["param"], to_dev(wl.init_weight(w, 5), "bf16"))


def test_ns_output_refused_after_fused_step():
    w = _mixed_shapes()
    ents = build_entries(w, normuon=False)
    plan = api.Plan(ents, api.make_hparams())
    for i, (e, p) in enumerate(zip(ents, w.params)):
        e["grad"].copy_(to_dev(wl.grad(w, i, 1), p.dtype))
    plan.step()
    torch.cuda.synchronize()
    with pytest.raises(L.LibraryError):
        plan.ns_output(0)
    plan.keep_ns_output(True)
    plan.step()
    torch.cuda.synchronize()
    assert plan.ns_output(0).shape == (96, 256)


def _aligned_shapes():
    """Slices whose iteration 0 reads D in place (wide or square, the long
    side a multiple of the tile; a padded short side reads zero past its last
    row) beside ones that keep the prep copy (tall, also from fp32 gradients
    and inside a view; a long side off the tile)."""
    ps = [wl.ParamSpec("norm", (64,), "bf16", wl.ROLE_NORM, no_decay=True),
          wl.ParamSpec("square", (256, 256), "bf16"),
          wl.ParamSpec("wide", (256, 640), "bf16"),
          wl.ParamSpec("big", (512, 768), "bf16"),
          wl.ParamSpec("tall", (512, 256), "bf16"),
          wl.ParamSpec("tall_pair", (1024, 256), "bf16", view=(2, 512, 256)),
          wl.ParamSpec("tall_f32", (384, 256), "f32"),
          wl.ParamSpec("padded", (200, 336), "bf16"),
          wl.ParamSpec("short_pad", (192, 512), "bf16"),
          wl.ParamSpec("short_ragged", (200, 512), "bf16"),
          # slice-resident and read in place (128 rows, columns a multiple of 128)
          wl.ParamSpec("heads", (256, 512), "bf16", view=(2, 128, 512)),
          wl.ParamSpec("head_wide", (128, 1024), "bf16")]
    return wl.Workload("aligned_shapes", 13, tuple(ps), grad_std=1e-3)


@pytest.mark.parametrize("coeffs", ["cubic", "quintic"])
@pytest.mark.parametrize("exp2", [0, -35, 35, -60, 55])
def test_first_iteration_in_place_and_range_fallback(exp2, coeffs):
    """Iteration 0 reads the unscaled D in place, the normalisation scale
    folded into the products; a slice whose max|D| leaves [2^-50, 2^40] (here
    gradients scaled by 2^-60 or 2^55) falls back to the prepared X0 (batched
    GEMM) or to X0 = bf16(s D) formed in LDS (slice-resident kernel).  The
    Newton-Schulz output meets the oracle's bound at every scale; the quintic
    cases put the 512-row slice on 256 x 256 tiles."""
    w = _aligned_shapes()
    cf = wl.coeff_table(coeffs)
    ents = build_entries(w, normuon=False)
    plan = api.Plan(ents, api.make_hparams(coeffs=cf),
                    options={"big_tile_min_work": 0 if coeffs == "quintic" else 512})
    plan.keep_ns_output(True)
    for i, (e, p) in enumerate(zip(ents, w.params)):
        e["grad"].copy_(to_dev(wl.grad(w, i, 1), p.dtype))
        e["grad"].mul_(2.0 ** exp2)     # a power of two: exact in bf16
    G = [f64(e["grad"]) for e in ents]
    plan.step()
    torch.cuda.synchronize()
    for k, (param, off, r, c) in enumerate(plan.slices()):
        _, D = omuon.momentum(np.zeros_like(G[param]), G[param], wl.MUON_MU)
        O_ref = omuon.newton_schulz(D[off:off + r], cf)
        assert_ns_close(f64(plan.ns_output(k)), O_ref, "bf16")


@pytest.mark.parametrize("steps", [1, 2, 3, 7])
@pytest.mark.parametrize("mode", ["gram_space", "plain"])
@pytest.mark.parametrize("row", ["cubic", "quintic"])
def test_iteration_count_and_mode(steps, mode, row):
    """The grouped step's Newton-Schulz output for 1, 2, 3 and 7 iterations,
    in Gram space (the default for the bf16 path: cubic rows on the GEMM
    path, any rows in the slice-resident kernel for short sides >= 64) and in
    the plain iteration (gram_space option off), against the oracle, over GEMM
    slices on both tile sizes and slice-resident slices on both sides of the
    64-row threshold."""
    opts = {"gram_space": mode == "gram_space", "big_tile_min_work": 0}
    base = _aligned_shapes()
    extra = [wl.ParamSpec("small_wide", (96, 256), "bf16"),
             wl.ParamSpec("small_tall", (392, 120), "bf16"),
             wl.ParamSpec("kv", (80, 64), "bf16", view=(2, 40, 64), split=(16, 24))]
    w = wl.Workload("iteration_shapes", 17, base.params + tuple(extra), grad_std=1e-3)
    cf = [(1.5, -0.5, 0.0) if row == "cubic" else (15 / 8, -5 / 4, 3 / 8)] * steps
    ents = build_entries(w, normuon=False)
    plan = api.Plan(ents, api.make_hparams(coeffs=cf), options=opts)
    plan.keep_ns_output(True)
    for i, (e, p) in enumerate(zip(ents, w.params)):
        e["grad"].copy_(to_dev(wl.grad(w, i, 1), p.dtype))
    G = [f64(e["grad"]) for e in ents]
    plan.step()
    torch.cuda.synchronize()
    for k, (param, off, r, c) in enumerate(plan.slices()):
        _, D = omuon.momentum(np.zeros_like(G[param]), G[param], wl.MUON_MU)
        assert_ns_close(f64(plan.ns_output(k)), omuon.newton_schulz(D[off:off + r], cf), "bf16")


# the per-iteration tables of the schedule tests: eight distinct cubic-type
# rows; cubic- and quintic-type rows mixed, identity rows (b = 0) included
_SCHED8 = [(a, 1.0 - a, 0.0) for a in (2.0, 1.0, 1.8, 1.1, 1.6, 1.2, 1.4, 1.0)]
_Q = (15 / 8, -10 / 8, 3 / 8)
_MIXED6 = [(2.0, -1.0, 0.0), (1.0, 0.0, 0.0), _Q, (1.3, -0.3, 0.0), _Q, (1.0, 0.0, 0.0)]


@pytest.mark.parametrize("row", ["cubic", "quintic", "sched8", "mixed6"])
@pytest.mark.parametrize("big", [False, True])
def test_gram_space_e_term_from_the_left_operand(row, big):
    """Gram-space products with an E term (T = a A + b A A, A' = a T + b T A,
    Q' = a Q + b Q A, the quintic P = b A + c A A + a I) take E from the left
    operand's slabs as they pass through LDS, in launches of many tiles (rows
    with b = 0 read E instead).  With the few-tile variant off, launches of
    these small shapes take that path: the Newton-Schulz output against the
    oracle, on both tile sizes, for repeated and per-iteration tables."""
    opts = {"few_tile_max": 0, "big_tile_min_work": 0 if big else -1}
    ps = [wl.ParamSpec("wide", (256, 640), "bf16"),
          wl.ParamSpec("big", (512, 1280), "bf16"),
          wl.ParamSpec("tall", (768, 256), "bf16"),
          wl.ParamSpec("padded", (200, 336), "bf16")]
    w = wl.Workload("e_term_shapes", 19, tuple(ps), grad_std=1e-3)
    cf = {"cubic": wl.coeff_table("cubic"), "quintic": wl.coeff_table("quintic"),
          "sched8": _SCHED8, "mixed6": _MIXED6}[row]
    ents = build_entries(w, normuon=False)
    plan = api.Plan(ents, api.make_hparams(coeffs=cf), options=opts)
    plan.keep_ns_output(True)
    algos = plan.slice_algorithms()
    assert all(a is not None and a[0] for a in algos)   # every slice in Gram space
    for i, (e, p) in enumerate(zip(ents, w.params)):
        e["grad"].copy_(to_dev(wl.grad(w, i, 1), p.dtype))
    G = [f64(e["grad"]) for e in ents]
    plan.step()
    torch.cuda.synchronize()
    for k, (param, off, r, c) in enumerate(plan.slices()):
        _, D = omuon.momentum(np.zeros_like(G[param]), G[param], wl.MUON_MU)
        print(f"[e-term] {row} big={big} slice {k} ({r}, {c})", flush=True)
        assert_ns_close(f64(plan.ns_output(k)), omuon.newton_schulz(D[off:off + r], cf), "bf16")


@pytest.mark.parametrize("normuon,precision", [(False, "bf16"), (True, "bf16"), (False, "fp32")],
                         ids=["plain", "normuon", "plain_fp32ns"])
def test_grouped_excluded_pieces(normuon, precision):
    """Fused weights with excluded pieces (Qwen3.8 optimizer notes, section 4):
    the excluded rows take the AdamW step (joint clip, the weight's step
    counter) and Muon leaves their momentum and weight rows alone; the other
    pieces take the Muon step."""
    w = wl.fused_exclude()
    ents = build_entries(w, normuon=normuon)
    coeffs = wl.coeff_table("cubic")
    plan = api.Plan(ents, api.make_hparams(coeffs=coeffs, normuon=normuon,
                                           ns_precision=precision))
    tol_ns = NS_F32_MAXABS if precision == "fp32" else NS_BF16_MAXABS
    descs = oracle_descs(w)
    st = HybridState()
    hp = HyperParams(coeffs=coeffs, normuon=normuon)
    Wref = {p.name: f64(e["param"]) for p, e in zip(w.params, ents)}
    norm = torch.zeros(1, dtype=torch.float64, device="cuda")
    for step in (1, 2, 3):
        G = {}
        for i, (p, e) in enumerate(zip(w.params, ents)):
            g = wl.grad(w, i, step)
            e["grad"].copy_(to_dev(g, p.dtype))
            G[p.name] = wl.from_storage(g, p.dtype).astype(np.float64)
        Wold = {p.name: f64(e["param"]) for p, e in zip(w.params, ents)}
        vold = {p.name: f64(e["normuon_v"]) for p, e in zip(w.params, ents) if "normuon_v" in e}
        plan.step(norm_out=norm)
        torch.cuda.synchronize()
        print(f"[excluded pieces] normuon={normuon} ns={precision} step {step}", flush=True)
        out = hybrid_step(descs, Wref, G, st, hp, keep_outputs=True)
        assert abs(f64(norm)[0] - out["T"]) <= 1e-12 * out["T"]
        for p, e in zip(w.params, ents):
            got = f64(e["param"])
            if p.name in out["muon"]:
                res = out["muon"][p.name]
                mine, excl = expand_pieces(p.shape, p.view, p.split, p.exclude)
                mom = f64(e["momentum"])
                dgot, dref = got - Wold[p.name], -0.01 * res["U"]
                pi = w.index(p.name)
                for off, r, c in mine:
                    rows = slice(off, off + r)
                    assert rel_inf(mom[rows], res["B"][rows]) <= REL_F32
                    sc = math.sqrt(max(1.0, r / c))
                    if normuon:
                        # the row step amplifies the Newton-Schulz rounding, so
                        # it is checked on the GPU's own O (which is checked
                        # against the oracle's)
                        k = plan.slices().index((pi, off, r, c))
                        O = f64(plan.ns_output(k))
                        assert_ns_close(O, res["O"][rows], "bf16")
                        On, v_exp = omuon.normuon_rownorm(O, vold[p.name][rows],
                                                          hp.normuon_beta2, hp.normuon_eps)
                        assert rel_inf(f64(e["normuon_v"])[rows], v_exp) <= 1e-5
                        assert_bf16_close(got[rows],
                                          omuon.apply_update(Wold[p.name][rows], sc * On, 0.01),
                                          extra=2e-6 * 0.01 * sc * np.abs(On))
                        continue
                    err = np.abs(dgot[rows] - dref[rows]).max()
                    ulp = bf16_ulp(Wold[p.name][rows]).max()
                    assert err <= 0.01 * sc * tol_ns + ulp, (p.name, off, err)
                for off, r, c in excl:
                    rows = slice(off, off + r)
                    assert not mom[rows].any(), (p.name, off)
                    want = out["W"][p.name][rows]
                    assert np.all(np.abs(got[rows] - want) <= bf16_ulp(want)), (p.name, off)
                    assert rel_inf(f64(e["exp_avg"])[rows], st.m[p.name][rows]) <= REL_F32
                    assert rel_inf(f64(e["exp_avg_sq"])[rows], st.v[p.name][rows]) <= REL_F32
                if excl:
                    kept = np.ones(p.shape[0], bool)
                    for off, r, _ in excl:
                        kept[off:off + r] = False
                    assert not f64(e["exp_avg"])[kept].any()
            else:
                want = out["W"][p.name]
                assert np.all(np.abs(got - want) <= bf16_ulp(want)), p.name
                assert rel_inf(f64(e["exp_avg"]), st.m[p.name]) <= REL_F32
                assert rel_inf(f64(e["exp_avg_sq"]), st.v[p.name]) <= REL_F32
            Wref[p.name] = got.copy()
    assert plan.get_steps() == [3, 3, 0, 3]
