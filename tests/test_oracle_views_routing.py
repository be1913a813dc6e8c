"""Pins for the oracle's view expansion and routing (CPU only)."""

import json
import os

import numpy as np
import pytest

import workloads as wl
from oracle import routing, views

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _load("view_examples.json")["cases"], ids=lambda c: c["name"])
def test_view_examples_from_page(case):
    sl = views.expand(tuple(case["stored"]), case["view"], case["split"])
    assert [list(s) for s in sl] == case["slices"]
    assert [[r, c] for _, r, c in sl] == case["independent_shapes"]


@pytest.mark.parametrize("case", _load("view_examples.json")["cases"], ids=lambda c: c["name"])
def test_view_expansion_matches_bruteforce_reshape(case):
    R, C = case["stored"]
    idx = np.arange(R * C).reshape(R, C)
    mats = idx.reshape(case["view"]).reshape(-1, case["view"][-2], C)
    want = []
    for m in mats:
        rows = m[:, 0] // C
        if case["split"]:
            start = 0
            for q in case["split"]:
                want.append((int(rows[start]), q, C))
                start += q
        else:
            want.append((int(rows[0]), len(rows), C))
    assert views.expand((R, C), case["view"], case["split"]) == want


def test_kda_leading_index_is_q_major():
    # (3, H, D, C): leading index q*H + h; Q head 0 = rows 0-3, K head 0 = rows 8-11.
    sl = views.expand((24, 8), (3, 2, 4, 8))
    assert sl[0] == (0, 4, 8) and sl[2] == (8, 4, 8)


@pytest.mark.parametrize("stored,view,split", [
    ((32, 8), (2, 15, 8), None),       # product mismatch
    ((32, 8), (2, 16, 7), None),       # cols mismatch
    ((32, 8), (0, 16, 8), None),       # non-positive entry
    ((32, 8), (2.0, 16, 8), None),     # not an int
    ((20, 8), (2, 10, 8), (4, 5)),     # split does not sum to rows
    ((20, 8), (2, 10, 8), (4, 0, 6)),  # split entry not positive
    ((20, 8), None, (4, 6)),           # split without a view
])
def test_invalid_views_refused(stored, view, split):
    with pytest.raises(views.ViewError):
        views.expand(stored, view, split)


def test_no_view_is_one_slice():
    assert views.expand((7, 5)) == [(0, 7, 5)]


def test_tiny_routing_groups():
    w = wl.tiny_routing()
    g = routing.build_groups(routing.descs_from_specs(w.params))
    keys = [x["key"] for x in g]
    assert keys == [
        ("adamw", None, None, False),
        ("muon", (2, 16, 8), None, True),
        ("muon", (3, 2, 4, 8), None, True),
        ("muon", (2, 10, 8), (4, 6), True),
    ]
    assert g[0]["names"] == ["embed_tokens.weight", "norm.weight"]


def test_omn1_counts_from_page():
    gold = _load("omn1_counts.json")
    g = routing.build_groups(routing.descs_from_specs(wl.omn1_shapes()))
    specs = {p.name: p for p in wl.omn1_shapes()}
    muon = [n for x in g if x["algorithm"] == "muon" for n in x["names"]]
    adam = [n for x in g if x["algorithm"] == "adamw" for n in x["names"]]
    decay_adam = [n for x in g if x["algorithm"] == "adamw" and x["decay"] for n in x["names"]]
    assert len(muon) == gold["muon_tensors"]
    assert sum(specs[n].numel for n in muon) == gold["muon_params"]
    assert sum(specs[n].numel for n in adam) == gold["adamw_params"]
    assert sum(p.numel for p in wl.omn1_shapes()) == gold["total_params"]
    assert len(decay_adam) == gold["adamw_decay_group_tensors"]
    blk = [specs[n].numel for n in muon if n.startswith("blocks.0.")]
    assert sum(blk) == gold["per_block_muon"]
    attn = sum(specs[n].numel for n in muon if n.startswith("blocks.0.attn"))
    assert attn == gold["per_block_attention"]
    assert sum(blk) - attn == gold["per_block_ffn"]
    assert specs["embed_tokens.weight"].numel == gold["embedding_params"]


def test_tied_weight_visited_once():
    d = [{"name": "embed_tokens.weight", "shape": (64, 8), "role": "embedding", "no_decay": True,
          "ident": 7},
         {"name": "q.weight", "shape": (8, 8), "ident": 1},
         {"name": "lm_head.weight", "shape": (64, 8), "role": "head", "ident": 7}]
    g = routing.build_groups(d)
    names = [n for x in g for n in x["names"]]
    assert names == ["embed_tokens.weight", "q.weight"]


def test_frozen_skipped_and_empty_raises():
    d = [{"name": "a", "shape": (4, 4), "requires_grad": False}]
    with pytest.raises(ValueError):
        routing.build_groups(d)
    d.append({"name": "b", "shape": (4,)})
    g = routing.build_groups(d)
    assert g[0]["names"] == ["b"]


def test_three_d_goes_to_decayed_adamw():
    d = [{"name": "conv.weight", "shape": (8, 1, 4)}, {"name": "head.weight", "shape": (4, 8),
                                                      "role": "head"}]
    g = routing.build_groups(d)
    assert g[0]["key"] == ("adamw", None, None, True)
    assert g[0]["names"] == ["conv.weight", "head.weight"]


def test_conflicting_views_refused():
    d = [{"name": "w", "shape": (32, 8), "ident": 3, "view": (2, 16, 8)},
         {"name": "w_alias", "shape": (32, 8), "ident": 3, "view": (4, 8, 8)}]
    with pytest.raises(ValueError):
        routing.build_groups(d)


def test_dense_and_head_batched_counts():
    w = wl.dense_decoder()
    g = routing.build_groups(routing.descs_from_specs(w.params))
    specs = {p.name: p for p in w.params}
    muon = [n for x in g if x["algorithm"] == "muon" for n in x["names"]]
    adam = [n for x in g if x["algorithm"] == "adamw" for n in x["names"]]
    assert len(muon) == 168 and sum(specs[n].numel for n in muon) == 1_233_125_376
    assert len(adam) == 50 and sum(specs[n].numel for n in adam) == 262_768_640
    f = wl.dense_decoder(fused_gate_up=True, normuon=True)
    gf = routing.build_groups(routing.descs_from_specs(f.params))
    fs = {p.name: p for p in f.params}
    nsl = sum(len(views.expand(fs[n].shape, x["view"], x["split"]))
              for x in gf if x["algorithm"] == "muon" for n in x["names"])
    assert nsl == 168
    h = wl.head_batched()
    gh = routing.build_groups(routing.descs_from_specs(h.params))
    hs = {p.name: p for p in h.params}
    nsl = sum(len(views.expand(hs[n].shape, x["view"], x["split"]))
              for x in gh for n in x["names"])
    assert nsl == 3072
    assert sum(p.numel for p in h.params) == 1_023_410_176
