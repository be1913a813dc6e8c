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


def _mixed_vs_separate(steps=2):
    """A fused (H * 3r, C) weight with view (H, 3r, C), split (r, r, r) and
    piece 1 excluded, against the same rows as separate weights: each Muon
    piece a plain Muon weight, each excluded piece an AdamW weight that
    decays (the decay flag a fused Muon weight carries)."""
    rng = np.random.default_rng(7)
    H, r, C = 2, 8, 12
    hp = HyperParams(muon_wd=0.1, adamw_wd=0.05, adamw_lr=3e-3)
    fused = [{"name": "f", "shape": (H * 3 * r, C), "view": (H, 3 * r, C), "split": (r, r, r),
              "exclude": (1,), "dtype": "f32"},
             {"name": "n", "shape": (C,), "dtype": "f32"}]
    sep = [{"name": "n", "shape": (C,), "dtype": "f32"}]
    rows = []
    for h in range(H):
        for j in range(3):
            nm = f"p{h}{j}"
            rows.append((nm, (h * 3 + j) * r))
            sep.append({"name": nm, "shape": (r, C), "dtype": "f32",
                        "role": "head" if j == 1 else "matrix"})
    Wf = {"f": bf16.round_to(rng.standard_normal((H * 3 * r, C)), "f32"),
          "n": bf16.round_to(rng.standard_normal(C), "f32")}
    Ws = {"n": Wf["n"]}
    Ws.update({nm: Wf["f"][o:o + r] for nm, o in rows})
    sf, ss = HybridState(), HybridState()
    for step in range(steps):
        Gf = {"f": rng.standard_normal((H * 3 * r, C)) * (step + 1),
              "n": rng.standard_normal(C)}
        Gs = {"n": Gf["n"]}
        Gs.update({nm: Gf["f"][o:o + r] for nm, o in rows})
        of = hybrid_step(fused, Wf, Gf, sf, hp)
        os_ = hybrid_step(sep, Ws, Gs, ss, hp)
        Wf, Ws = of["W"], os_["W"]
        yield of, os_, sf, ss, rows, r


def test_excluded_pieces_equal_separate_weights():
    # Pin: gathering the pieces back into the fused layout changes nothing
    # (Qwen3.8 notes, section 4), so the fused step with excluded pieces must
    # equal the step over the pieces as weights of their own.
    for of, os_, sf, ss, rows, r in _mixed_vs_separate():
        assert math.isclose(of["T"], os_["T"], rel_tol=1e-14)
        assert math.isclose(of["kappa"], os_["kappa"], rel_tol=1e-14)
        for nm, o in rows:
            np.testing.assert_allclose(of["W"]["f"][o:o + r], os_["W"][nm], rtol=1e-6, atol=0)
            if nm.endswith("1"):
                np.testing.assert_allclose(sf.m["f"][o:o + r], ss.m[nm], rtol=1e-12)
                np.testing.assert_allclose(sf.v["f"][o:o + r], ss.v[nm], rtol=1e-12)
                assert not sf.B["f"][o:o + r].any()    # Muon never touched these rows
            else:
                np.testing.assert_allclose(sf.B["f"][o:o + r], ss.B[nm], rtol=1e-12)
                assert not sf.m["f"][o:o + r].any()
        assert sf.t["f"] == ss.t["p01"]


def test_exclude_validation():
    import pytest
    from oracle.routing import build_groups
    base = {"name": "f", "shape": (24, 8), "view": (2, 12, 8), "split": (4, 8)}
    for bad in ({"exclude": (2,)}, {"exclude": (0, 1)}, {"split": None, "exclude": (0,)}):
        with pytest.raises(ValueError):
            build_groups([dict(base, **bad)])
    g = build_groups([dict(base, exclude=(1,)), dict(base, name="g", exclude=(0,)),
                      dict(base, name="h")])
    assert [x["exclude"] for x in g] == [(1,), (0,), None]
