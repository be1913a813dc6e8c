"""Full-size parity: the grouped hybrid step at the workloads' real sizes, built
by the same plan builder and run in the same launch configuration that the
benchmark times, checked against the fp64 oracle.

Whole-matrix checks where the oracle finishes in seconds (the single-matrix
Newton-Schulz sweep); elsewhere sampled slices (every distinct shape, first and
last layers) that the oracle computes one by one, the exact global clip norm
over every AdamW gradient, sampled AdamW elements, and properties that hold for
every slice at any size.

The Newton-Schulz output O of a slice is read from the workspace with
mo_plan_ns_output (the point before NorMuon, shape scale and learning rate).
"""

import math

import numpy as np
import pytest
import torch

import bench
import workloads as wl
from adamw_optimizer_step_amd import _lib as L
from oracle import adamw as oadamw
from oracle import muon as omuon
from oracle.views import expand

from gpu_common import (NS_BF16_MAXABS, REL_F32, assert_bf16_close, assert_ns_close, bf16_ulp,
                        f64, rel_inf, require_gpu)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _run(w, coeffs_kind, precision, sample_params, spectral_cap=0.0, spectral_iters=8):
    """Build the benchmark's plan for `w`, keep host copies of what the checks
    need, run one step with O kept in the workspace.  Returns (plan, entries,
    routes, before, T_gpu); before["muon_w0"] holds device copies of every
    Muon weight as it was before the step."""
    coeffs = wl.coeff_table(coeffs_kind, w.ns_steps)
    plan, ents, routes = bench.build_plan(w, coeffs, precision, w.normuon, spectral_cap,
                                          spectral_iters)
    plan.keep_ns_output(True)      # the checks read O from the workspace
    ws = plan.workspace(torch.device("cuda"))
    before = {"muon_w0": {i: e["param"].clone() for i, (e, r) in enumerate(zip(ents, routes))
                          if r[0] == L.MO_ALG_MUON}}
    for i in sample_params:
        before[i] = {"W": f64(ents[i]["param"]), "G": f64(ents[i]["grad"])}
    norm = torch.zeros(1, dtype=torch.float64, device="cuda")
    torch.cuda.synchronize()
    print(f"[fullsize] {w.key} {coeffs_kind} {precision}: step", flush=True)
    plan.step(workspace=ws, norm_out=norm)
    torch.cuda.synchronize()
    return plan, ents, routes, before, float(norm.item()), coeffs


def _fused_equals_kept(plan, ents, before):
    """Repeat the step from the same Muon weights and zero momentum, now in
    the benchmark's default mode (the update inside the last Newton-Schulz
    launch): every Muon weight equals the kept-O step's bit for bit."""
    kept = {}
    for i, w0 in before["muon_w0"].items():
        kept[i] = ents[i]["param"].clone()
        ents[i]["param"].copy_(w0)
        ents[i]["momentum"].zero_()
    plan.keep_ns_output(False)
    assert plan.fuses_update()
    torch.cuda.synchronize()
    print("[fullsize] fused step", flush=True)
    plan.step()
    torch.cuda.synchronize()
    for i, k in kept.items():
        assert torch.equal(ents[i]["param"], k), i


def _slice_index(plan, param, off):
    for k, (p, o, _, _) in enumerate(plan.slices()):
        if p == param and o == off:
            return k
    raise KeyError((param, off))


def _check_muon_param(w, plan, ents, i, before, coeffs, precision, lr=wl.MUON_LR,
                      slices_to_check=None):
    """Oracle Muon step of param i (B0 = 0, step 1) against the GPU: momentum,
    NS output per slice, NorMuon state and the new weight."""
    p = w.params[i]
    sl = expand(p.shape, p.view, p.split)
    G, W0 = before[i]["G"], before[i]["W"]
    B_gpu = f64(ents[i]["momentum"])
    B_ref, D_ref = omuon.momentum(np.zeros_like(G), G, wl.MUON_MU)
    assert rel_inf(B_gpu, B_ref) <= REL_F32
    W_gpu = f64(ents[i]["param"])
    v_gpu = f64(ents[i]["normuon_v"]) if w.normuon else None
    chosen = sl if slices_to_check is None else [sl[k] for k in slices_to_check]
    for off, r, c in chosen:
        k = _slice_index(plan, i, off)
        O_gpu = f64(plan.ns_output(k))
        O_ref = omuon.newton_schulz(D_ref[off:off + r], coeffs)
        assert_ns_close(O_gpu, O_ref, precision)
        scale = omuon.shape_scale(r, c)
        U_gpu = O_gpu
        if w.normuon:
            # row state from the GPU's own O (isolates the row kernel), and
            # against the oracle's O within the NS tolerance
            On, v_exp = omuon.normuon_rownorm(O_gpu, np.zeros(r), wl.NORMUON_BETA2,
                                              wl.NORMUON_EPS)
            vs = v_gpu[off:off + r]
            # fp32 row sums of up to 5632 squares: a few 1e-7 relative
            assert rel_inf(vs, v_exp) <= 1e-5
            _, v_ref = omuon.normuon_rownorm(O_ref, np.zeros(r), wl.NORMUON_BETA2,
                                             wl.NORMUON_EPS)
            assert rel_inf(vs, v_ref) <= 5e-2
            U_gpu = On
        Ws = W_gpu[off:off + r]
        # exact given the GPU's O: W0 - lr scale U rounded to bf16 (one ulp)
        W_exp = omuon.apply_update(W0[off:off + r], scale * U_gpu, lr)
        if p.dtype == "bf16":
            assert_bf16_close(Ws, W_exp, extra=2e-6 * lr * scale * np.abs(U_gpu))
        else:
            assert rel_inf(Ws, W_exp) <= REL_F32
        if not w.normuon:
            W_ref = omuon.apply_update(W0[off:off + r], scale * O_ref, lr)
            bound = lr * scale * NS_BF16_MAXABS + bf16_ulp(W_ref)
            assert np.all(np.abs(Ws - W_ref) <= bound)


def _check_adamw(w, ents, routes, before, T_gpu, sample_params, rng):
    """Global clip norm over every AdamW gradient (exact, fp64), then sampled
    AdamW elements of the sampled params at step 1."""
    chunks = []
    for i, r in enumerate(routes):
        if r[0] != L.MO_ALG_ADAMW:
            continue
        g = ents[i]["grad"].float().cpu().numpy().reshape(-1)
        chunks.extend(g[j:j + (1 << 22)] for j in range(0, g.size, 1 << 22))
    T = oadamw.global_norm(chunks)
    assert abs(T_gpu - T) <= 1e-9 * T, (T_gpu, T)
    kappa = oadamw.clip_factor(T, wl.CLIP_MAX_NORM)
    for i in sample_params:
        if routes[i][0] != L.MO_ALG_ADAMW:
            continue
        G = before[i]["G"].reshape(-1)
        W0 = before[i]["W"].reshape(-1)
        idx = np.arange(G.size) if G.size <= (1 << 16) else \
            np.sort(rng.choice(G.size, size=1 << 16, replace=False))
        W_ref, m_ref, v_ref = oadamw.adamw_update(
            W0[idx], G[idx], 0.0, 0.0, 1, wl.ADAMW_LR, wl.ADAMW_BETA1, wl.ADAMW_BETA2,
            wl.ADAMW_EPS, 0.0, kappa)
        m = f64(ents[i]["exp_avg"]).reshape(-1)[idx]
        v = f64(ents[i]["exp_avg_sq"]).reshape(-1)[idx]
        Wn = f64(ents[i]["param"]).reshape(-1)[idx]
        assert rel_inf(m, m_ref) <= REL_F32
        assert rel_inf(v, v_ref) <= REL_F32
        assert_bf16_close(Wn, W_ref)


def _all_slices_bounded(plan, precision):
    """Every slice's O is finite and ||O||_F <= sqrt(short side) (1 + 2e-2):
    each polynomial maps [0, 1] into [0, 1], so all singular values stay at
    most one up to rounding."""
    for k, (_, _, r, c) in enumerate(plan.slices()):
        O = plan.ns_output(k).float()
        fro = float(torch.linalg.vector_norm(O))
        assert math.isfinite(fro), k
        assert fro <= math.sqrt(min(r, c)) * (1 + 2e-2), (k, fro)


@pytest.mark.parametrize("rows,cols", [(1024, 1024), (4096, 1024)])
@pytest.mark.parametrize("coeffs", ["cubic", "quintic"])
def test_ns_sweep_full(rows, cols, coeffs):
    w = wl.ns_sweep(rows, cols, coeffs)
    plan, ents, routes, before, _, cf = _run(w, coeffs, "bf16", [0])
    _check_muon_param(w, plan, ents, 0, before, cf, "bf16")
    _fused_equals_kept(plan, ents, before)


def test_ns_sweep_fp32_path():
    w = wl.ns_sweep(4096, 1024, "cubic")
    plan, ents, routes, before, _, cf = _run(w, "cubic", "fp32", [0])
    G = before[0]["G"]
    _, D_ref = omuon.momentum(np.zeros_like(G), G, wl.MUON_MU)
    O_ref = omuon.newton_schulz(D_ref, cf)
    assert_ns_close(f64(plan.ns_output(0)), O_ref, "fp32")


def _dense_sample(w):
    names = ["layers.0.attn.q_proj.weight", "layers.23.attn.v_proj.weight",
             "layers.11.mlp.gate_proj.weight", "layers.23.mlp.down_proj.weight",
             "embed_tokens.weight", "layers.0.input_norm.weight", "final_norm.weight"]
    if w.normuon:
        names[2] = "layers.11.mlp.gate_up_proj.weight"
    return [w.index(n) for n in names]


@pytest.mark.parametrize("coeffs", ["cubic", "quintic"])
def test_dense_decoder_full(coeffs):
    w = wl.dense_decoder()
    sample = _dense_sample(w)
    plan, ents, routes, before, T_gpu, cf = _run(w, coeffs, "bf16", sample)
    assert len(plan.slices()) == 168
    for i in sample:
        if routes[i][0] == L.MO_ALG_MUON:
            _check_muon_param(w, plan, ents, i, before, cf, "bf16")
    _check_adamw(w, ents, routes, before, T_gpu, sample, np.random.default_rng(3))
    _all_slices_bounded(plan, "bf16")
    _fused_equals_kept(plan, ents, before)


def test_dense_decoder_fp32_path_full():
    """The dense decoder with the fp32 Newton-Schulz path (the OMN page's
    precision), sampled slices at the fp32 bound of 1e-4."""
    w = wl.dense_decoder()
    sample = _dense_sample(w)
    plan, ents, routes, before, T_gpu, cf = _run(w, "cubic", "fp32", sample)
    for i in sample:
        if routes[i][0] == L.MO_ALG_MUON:
            _check_muon_param(w, plan, ents, i, before, cf, "fp32")
    _check_adamw(w, ents, routes, before, T_gpu, sample, np.random.default_rng(6))
    _all_slices_bounded(plan, "fp32")


def test_dense_decoder_spectral_cap_full():
    """The dense decoder with the spectral-cap guard on (OMN page, Muon-path
    paragraph), built as the benchmark builds it: tau = 0.1 lies between the
    step-1 estimates of the square attention slices (about 0.09 for these
    gradients) and of the rectangular MLP slices (about 0.12), so the cap
    binds on some slices and not on others.  Sampled slices: the capped
    buffer against the oracle's (1e-6), the Newton-Schulz output from the
    capped D, and the weights given the GPU's own O."""
    w = wl.dense_decoder()
    tau, iters = 0.1, 8
    sample = _dense_sample(w)
    plan, ents, routes, before, T_gpu, cf = _run(w, "cubic", "bf16", sample, tau, iters)
    bound = 0
    for i in sample:
        if routes[i][0] != L.MO_ALG_MUON:
            continue
        p = w.params[i]
        G, W0 = before[i]["G"], before[i]["W"]
        B_gpu, W_gpu = f64(ents[i]["momentum"]), f64(ents[i]["param"])
        for off, r, c in expand(p.shape, p.view, p.split):
            rows = slice(off, off + r)
            B1, _ = omuon.momentum(np.zeros((r, c)), G[rows], wl.MUON_MU)
            sigma = omuon.spectral_estimate(B1, iters)
            bound += int(sigma > tau)
            B_ref = omuon.spectral_cap(B1, tau, iters)
            print(f"[fullsize] cap {p.name} rows {off}:{off + r} sigma {sigma:.4f}", flush=True)
            assert rel_inf(B_gpu[rows], B_ref) <= REL_F32, (p.name, off)
            D_ref = G[rows] + wl.MUON_MU * B_ref
            O_gpu = f64(plan.ns_output(_slice_index(plan, i, off)))
            assert_ns_close(O_gpu, omuon.newton_schulz(D_ref, cf), "bf16")
            sc = omuon.shape_scale(r, c)
            W_exp = omuon.apply_update(W0[rows], sc * O_gpu, wl.MUON_LR)
            assert_bf16_close(W_gpu[rows], W_exp, extra=2e-6 * wl.MUON_LR * sc * np.abs(O_gpu))
    assert 0 < bound < 4            # the cap bound on some sampled slices, not all
    _check_adamw(w, ents, routes, before, T_gpu, sample, np.random.default_rng(5))
    _all_slices_bounded(plan, "bf16")


def test_dense_decoder_fused_normuon_full():
    w = wl.dense_decoder(fused_gate_up=True, normuon=True)
    sample = _dense_sample(w)
    plan, ents, routes, before, T_gpu, cf = _run(w, "cubic", "bf16", sample)
    assert len(plan.slices()) == 168
    for i in sample:
        if routes[i][0] == L.MO_ALG_MUON:
            _check_muon_param(w, plan, ents, i, before, cf, "bf16")
    _check_adamw(w, ents, routes, before, T_gpu, sample, np.random.default_rng(4))
    # NorMuon's row statistics span whole rows: the separate row pass stays
    plan.keep_ns_output(False)
    assert not plan.fuses_update()


@pytest.mark.parametrize("coeffs", ["cubic", "quintic"])
def test_head_batched_full(coeffs):
    w = wl.head_batched()
    names = {"layers.0.attn.W_UQ.weight": [0, 31], "layers.15.attn.W_UQ.weight": [17],
             "layers.0.attn.W_UKV.weight": [0, 1, 63], "layers.15.attn.W_UKV.weight": [40],
             "layers.0.attn.QKV.weight": [0, 37, 95], "layers.15.attn.QKV.weight": [64]}
    sample = [w.index(n) for n in names]
    plan, ents, routes, before, _, cf = _run(w, coeffs, "bf16", sample)
    assert len(plan.slices()) == 3072
    for n, ks in names.items():
        i = w.index(n)
        _check_muon_param(w, plan, ents, i, before, cf, "bf16", slices_to_check=ks)
    _all_slices_bounded(plan, "bf16")
    _fused_equals_kept(plan, ents, before)
