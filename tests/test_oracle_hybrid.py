"""Whole-step pins for the oracle on the tiny routing workload (CPU only)."""

import math

import numpy as np

import workloads as wl
from oracle import bf16, muon
from oracle.hybrid import HybridState, HyperParams, hybrid_step
from oracle.routing import descs_from_specs


def _setup(w):
    descs = descs_from_specs(w.params)
    for d, p in zip(descs, w.params):
        d["dtype"] = p.dtype
    W = {p.name: bf16.widen(wl.init_weight(w, i), p.dtype) for i, p in enumerate(w.params)}
    return descs, W


def _grads(w, step):
    return {p.name: bf16.widen(wl.grad(w, i, step), p.dtype) for i, p in enumerate(w.params)}


def test_tiny_three_steps_clip_and_updates():
    w = wl.tiny_routing()
    descs, W = _setup(w)
    st = HybridState()
    hp = HyperParams()
    for step in (1, 2, 3):
        G = _grads(w, step)
        adam_names = ("embed_tokens.weight", "norm.weight")
        T_want = math.sqrt(sum(np.sum(G[n] ** 2) for n in adam_names))
        out = hybrid_step(descs, W, G, st, hp, keep_outputs=True)
        assert out["T"] == T_want and out["T"] > 1.0
        assert out["kappa"] == 1.0 / T_want
        for name, res in out["muon"].items():
            # update = -lr * scale * O per slice; here wd = 0 and fp32 rounding.
            np.testing.assert_allclose(out["W"][name], bf16.round_to(W[name] - 0.01 * res["U"],
                                                                     "f32"))
        W = out["W"]
        assert all(st.t[n] == step for n in adam_names)
    assert len(st.B) == 3


def test_muon_grads_do_not_change_clip():
    w = wl.tiny_routing()
    descs, W = _setup(w)
    G = _grads(w, 1)
    a = hybrid_step(descs, W, G, HybridState(), HyperParams())
    G2 = dict(G)
    G2["attn.QKV.weight"] = G["attn.QKV.weight"] * 1e6
    b = hybrid_step(descs, W, G2, HybridState(), HyperParams())
    assert a["kappa"] == b["kappa"] and a["T"] == b["T"]
    assert np.array_equal(a["W"]["norm.weight"], b["W"]["norm.weight"])


def test_param_without_grad_is_untouched():
    w = wl.tiny_routing()
    descs, W = _setup(w)
    G = _grads(w, 1)
    G["attn.W_UKV.weight"] = None
    G["norm.weight"] = None
    st = HybridState()
    out = hybrid_step(descs, W, G, st, HyperParams())
    assert np.array_equal(out["W"]["attn.W_UKV.weight"], W["attn.W_UKV.weight"])
    assert np.array_equal(out["W"]["norm.weight"], W["norm.weight"])
    assert "attn.W_UKV.weight" not in st.B and "norm.weight" not in st.t
    T = math.sqrt(np.sum(G["embed_tokens.weight"] ** 2))
    assert out["T"] == T


def test_ns_output_rows_per_slice_bounded():
    # The NS output after the normalisation has spectral norm <= 1 in exact
    # arithmetic for the cubic (p maps [0, 1] into [0, 1]).
    w = wl.tiny_routing()
    descs, W = _setup(w)
    out = hybrid_step(descs, W, _grads(w, 1), HybridState(), HyperParams(), keep_outputs=True)
    from oracle.views import expand
    specs = {p.name: p for p in w.params}
    for name, res in out["muon"].items():
        for off, r, c in expand(specs[name].shape, specs[name].view, specs[name].split):
            assert np.linalg.norm(res["O"][off:off + r], 2) <= 1.0 + 1e-12
    assert muon.shape_scale(16, 8) == math.sqrt(2.0)
