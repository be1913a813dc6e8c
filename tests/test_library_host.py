"""CPU tests of the C ABI library: loading, exported symbols, struct layout,
host-only routing / view expansion against the oracle, plan tables and
argument validation (every failing call returns before touching the GPU)."""

import ctypes as C
import os
import re

import numpy as np
import pytest

import workloads as wl
from adamw_optimizer_step_amd import _lib as L
from adamw_optimizer_step_amd import api
from oracle import routing as orouting
from oracle import views as oviews

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "muon_adamw.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set()
    for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M):
        line = text[m.start():m.end()]
        if line.startswith(("typedef", "#", "struct")):
            continue
        names.add(m.group(1))
    return sorted(names)


def test_library_loads_and_exports_every_declared_symbol():
    lib = L.lib()
    names = _declared_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(s[0] for s in L.SIGNATURES) == names
    assert lib.mo_version().startswith(b"muon_adamw")


def test_struct_layouts_match():
    for i, S in enumerate(L.ABI_STRUCTS):
        assert C.sizeof(S) == L.lib().mo_abi_struct_size(i), S.__name__
    assert L.lib().mo_abi_struct_size(99) == 0


def _descs_for(specs):
    return [api.make_desc(p.name, p.shape, p.role, p.no_decay, p.requires_grad, i, p.view,
                          p.split, p.exclude) for i, p in enumerate(specs)]


def _oracle_routes(specs):
    descs = orouting.descs_from_specs(specs)
    for i, d in enumerate(descs):
        d["ident"] = i
    groups = orouting.build_groups(descs)
    want = [(L.MO_ALG_SKIP, 0, -1, 0)] * len(specs)
    for gi, g in enumerate(groups):
        for idx in g["indices"]:
            alg = L.MO_ALG_MUON if g["algorithm"] == "muon" else L.MO_ALG_ADAMW
            nsl = len(oviews.expand_pieces(specs[idx].shape, g["view"], g["split"],
                                           g["exclude"])[0]) if alg == 1 else 0
            want[idx] = (alg, int(g["decay"]), gi, nsl)
    return want, len(groups)


@pytest.mark.parametrize("specs", [wl.tiny_routing().params, wl.dense_decoder().params,
                                   wl.dense_decoder(fused_gate_up=True, normuon=True).params,
                                   wl.head_batched().params, wl.omn1_shapes(),
                                   wl.fused_exclude().params],
                         ids=["tiny", "dense", "dense_fused", "head_batched", "omn1",
                              "fused_exclude"])
def test_route_bit_exact_with_oracle(specs):
    got, ng = api.route(_descs_for(specs))
    want, wng = _oracle_routes(specs)
    assert got == want and ng == wng


def test_route_tied_frozen_and_errors():
    d = [api.make_desc("embed", (64, 8), "embedding", True, ident=7),
         api.make_desc("q", (8, 8), ident=1),
         api.make_desc("head", (64, 8), "head", ident=7),
         api.make_desc("frozen", (8, 8), requires_grad=False, ident=2),
         api.make_desc("conv", (8, 1, 4), ident=3)]
    r, ng = api.route(d)
    assert [x[0] for x in r] == [L.MO_ALG_ADAMW, L.MO_ALG_MUON, L.MO_ALG_SKIP, L.MO_ALG_SKIP,
                                 L.MO_ALG_ADAMW]
    assert r[4][1] == 1 and r[0][1] == 0 and ng == 3
    with pytest.raises(L.LibraryError) as e:
        api.route([api.make_desc("a", (4, 4), requires_grad=False)])
    assert e.value.status == L.MO_EEMPTY
    with pytest.raises(L.LibraryError) as e:
        api.route([api.make_desc("w", (32, 8), ident=3, view=(2, 16, 8)),
                   api.make_desc("w2", (32, 8), ident=3, view=(4, 8, 8))])
    assert e.value.status == L.MO_ECONFLICT
    for view, split in (((2, 15, 8), None), ((0, 16, 8), None), ((2, 16, 8), (4, 4))):
        with pytest.raises(L.LibraryError) as e:
            api.route([api.make_desc("w", (32, 8), view=view, split=split)])
        assert e.value.status == L.MO_ESHAPE


@pytest.mark.parametrize("case", [((32, 8), (2, 16, 8), None), ((24, 8), (3, 2, 4, 8), None),
                                  ((20, 8), (2, 10, 8), (4, 6)), ((7, 5), None, None),
                                  ((8192, 512), (32, 256, 512), (128, 128)),
                                  ((12288, 4096), (3, 32, 128, 4096), None),
                                  ((60, 3), (2, 3, 10, 3), (1, 2, 7))])
def test_expand_view_bit_exact_with_oracle(case):
    stored, view, split = case
    assert api.expand_view(*stored, view, split) == oviews.expand(stored, view, split)


def _fake_ptr(k):
    return 0x10000000 + 4096 * k


def _fake_entries(specs, normuon=False):
    routes, _ = api.route(_descs_for(specs))
    ents = []
    for i, (p, r) in enumerate(zip(specs, routes)):
        e = {"desc": api.make_desc(p.name, p.shape, p.role, p.no_decay, p.requires_grad, i,
                                   p.view, p.split, p.exclude)}
        ents.append(e)
    arr = (L.Param * len(specs))()
    for i, (e, r) in enumerate(zip(ents, routes)):
        arr[i].desc = e["desc"]
        arr[i].param = _fake_ptr(8 * i)
        arr[i].grad = _fake_ptr(8 * i + 1)
        arr[i].dtype = L.MO_BF16 if specs[i].dtype == "bf16" else L.MO_F32
        arr[i].momentum = _fake_ptr(8 * i + 2)
        arr[i].normuon_v = _fake_ptr(8 * i + 3) if normuon else None
        arr[i].exp_avg = _fake_ptr(8 * i + 4)
        arr[i].exp_avg_sq = _fake_ptr(8 * i + 5)
    return arr


@pytest.mark.parametrize("w", [wl.tiny_routing(), wl.head_batched(layers=2),
                               wl.fused_exclude()],
                         ids=["tiny", "head_batched_2l", "fused_exclude"])
def test_plan_slice_table_host_only(w):
    arr = _fake_entries(w.params)
    h = C.c_void_p()
    hp = api.make_hparams()
    L.check("plan", L.lib().mo_plan_create(arr, len(w.params), C.byref(hp), None, C.byref(h)))
    try:
        k = L.lib().mo_plan_num_slices(h)
        out = (C.c_int64 * (4 * k))()
        L.check("slices", L.lib().mo_plan_slices(h, out, k))
        got = [tuple(out[4 * i:4 * i + 4]) for i in range(k)]
        want = []
        for i, p in enumerate(w.params):
            if len(p.shape) == 2 and p.role == "matrix":
                want += [(i, o, r, c) for o, r, c in
                         oviews.expand_pieces(p.shape, p.view, p.split, p.exclude)[0]]
        assert got == want
        assert L.lib().mo_plan_workspace_bytes(h) > 0
        steps = (C.c_int32 * len(w.params))()
        L.check("steps", L.lib().mo_plan_get_steps(h, steps, len(w.params)))
        assert list(steps) == [0] * len(w.params)
    finally:
        L.lib().mo_plan_destroy(h)


def test_plan_validation_errors():
    w = wl.tiny_routing()
    arr = _fake_entries(w.params)
    h = C.c_void_p()
    hp = api.make_hparams()
    hp.ns_steps = 0
    assert L.lib().mo_plan_create(arr, len(w.params), C.byref(hp), None, C.byref(h)) == L.MO_EINVAL
    hp = api.make_hparams(normuon=True)      # NorMuon without v buffers
    assert L.lib().mo_plan_create(arr, len(w.params), C.byref(hp), None, C.byref(h)) == L.MO_EINVAL
    hp = api.make_hparams()
    arr[1].momentum = None                   # Muon param without momentum
    assert L.lib().mo_plan_create(arr, len(w.params), C.byref(hp), None, C.byref(h)) == L.MO_EINVAL
    assert not h.value
    assert L.lib().mo_grouped_step(None, None, None, 0, None) == L.MO_EINVAL


def test_entry_point_validation_before_enqueue():
    lib = L.lib()
    # momentum: NULL momentum, misaligned pointer, small workspace
    it = (L.MomentumItem * 1)()
    it[0].grad, it[0].momentum, it[0].numel = _fake_ptr(1), None, 16
    assert lib.muon_momentum(it, 1, 0.95, 1, None, 0, None) == L.MO_EINVAL
    it[0].momentum = _fake_ptr(2) + 4
    assert lib.muon_momentum(it, 1, 0.95, 1, None, 0, None) == L.MO_EALIGN
    it[0].momentum = _fake_ptr(2)
    assert lib.muon_momentum(it, 1, 0.95, 1, None, 0, None) == L.MO_EWORKSPACE
    it[0].grad_dtype = 7
    assert lib.muon_momentum(it, 1, 0.95, 1, None, 0, None) == L.MO_EDTYPE
    # NS: empty shape, bad steps, bad coefficients, workspace
    ns = (L.NsItem * 1)()
    ns[0].inp, ns[0].out, ns[0].rows, ns[0].cols, ns[0].ld_in, ns[0].ld_out = (
        _fake_ptr(3), _fake_ptr(4), 0, 8, 8, 8)
    co = (C.c_float * 15)(*([1.5, -0.5, 0.0] * 5))
    assert lib.ns_orthogonalize_batched(ns, 1, co, 5, 0, None, None, 0, None) == L.MO_ESHAPE
    ns[0].rows = 4
    assert lib.ns_orthogonalize_batched(ns, 1, co, 0, 0, None, None, 0, None) == L.MO_EINVAL
    assert lib.ns_orthogonalize_batched(ns, 1, co, 5, 9, None, None, 0, None) == L.MO_EINVAL
    bad = (C.c_float * 15)(*([float("nan")] * 15))
    assert lib.ns_orthogonalize_batched(ns, 1, bad, 5, 0, None, None, 0, None) == L.MO_EINVAL
    # options out of range
    opt = L.NsOptions()
    lib.mo_ns_options_default(C.byref(opt))
    assert (opt.gram_space, opt.big_tile_min_work, opt.few_tile_max) == (1, -1, -1)
    opt.gram_space = 2
    assert lib.ns_orthogonalize_batched(ns, 1, co, 5, 0, C.byref(opt), None, 0, None) == \
        L.MO_EINVAL
    opt.gram_space, opt.few_tile_max = 1, -2
    assert lib.ns_orthogonalize_batched(ns, 1, co, 5, 0, C.byref(opt), None, 0, None) == \
        L.MO_EINVAL
    need = lib.ns_workspace_bytes(ns, 1, None, 0, 0, None)   # the most any table needs
    assert need > 0
    qu = (C.c_float * 15)(*([15 / 8, -10 / 8, 3 / 8] * 5))
    assert lib.ns_workspace_bytes(ns, 1, qu, 5, 0, None) <= need
    assert lib.ns_workspace_bytes(ns, 1, co, 5, 0, None) <= need
    need_q = lib.ns_workspace_bytes(ns, 1, qu, 5, 0, None)
    assert lib.ns_orthogonalize_batched(ns, 1, qu, 5, 0, None, C.c_void_p(_fake_ptr(9)),
                                        need_q - 256, None) == L.MO_EWORKSPACE
    assert lib.ns_orthogonalize_batched(ns, 1, co, 5, 0, None, C.c_void_p(_fake_ptr(9) + 16),
                                        need, None) == L.MO_EALIGN
    ns[0].ld_in = 4
    assert lib.ns_orthogonalize_batched(ns, 1, co, 5, 0, None, None, 0, None) == L.MO_ESHAPE
    # AdamW: step 0, bad betas, workspace
    ad = (L.AdamwItem * 1)()
    ad[0].param, ad[0].grad, ad[0].exp_avg, ad[0].exp_avg_sq = [_fake_ptr(k) for k in (5, 6, 7, 8)]
    ad[0].numel, ad[0].dtype, ad[0].step = 100, L.MO_BF16, 0
    assert lib.adamw_clip_step(ad, 1, 1e-3, 0.9, 0.95, 1e-8, 1.0, None, None, 0, None) == L.MO_EINVAL
    ad[0].step = 1
    assert lib.adamw_clip_step(ad, 1, 1e-3, 1.0, 0.95, 1e-8, 1.0, None, None, 0, None) == L.MO_EINVAL
    assert lib.adamw_clip_step(ad, 1, 1e-3, 0.9, 0.95, 1e-8, 1.0, None, None, 0, None) == \
        L.MO_EWORKSPACE
    # row kernels
    assert lib.normuon_rownorm(None, 0, 4, 4, 4, None, 0.95, 1e-8, None) == L.MO_EINVAL
    assert lib.normuon_rownorm(_fake_ptr(1), 0, 4, 4, 3, _fake_ptr(2), 0.95, 1e-8, None) == \
        L.MO_ESHAPE
    assert lib.muon_update(_fake_ptr(1), 3, _fake_ptr(2), 0, 4, 4, 4, 4, 0.1, 0.0, 1.0, None) == \
        L.MO_EDTYPE
    assert lib.mo_last_error()  # message recorded


def _fuses(specs, normuon=False, precision="bf16", keep=False, offset=0):
    arr = _fake_entries(specs, normuon=normuon)
    if offset:   # Muon weights only (AdamW pointers must be aligned)
        for i, sp in enumerate(specs):
            if len(sp.shape) == 2:
                arr[i].param = _fake_ptr(8 * i) + offset
    h = C.c_void_p()
    hp = api.make_hparams(ns_precision=precision, normuon=normuon)
    L.check("plan", L.lib().mo_plan_create(arr, len(specs), C.byref(hp), None, C.byref(h)))
    try:
        if keep:
            L.check("keep", L.lib().mo_plan_keep_ns_output(h, 1))
        return L.lib().mo_plan_fuses_update(h)
    finally:
        L.lib().mo_plan_destroy(h)


def test_fused_update_eligibility():
    """The Muon update runs inside the last Newton-Schulz launch only for the
    bf16 path without NorMuon, with 16-byte weight chunks, unless O is kept."""
    ok = [wl.ParamSpec("w", (64, 48), "bf16"), wl.ParamSpec("t", (96, 16), "f32"),
          wl.ParamSpec("g", (16,), "bf16", role=wl.ROLE_NORM)]
    assert _fuses(ok) == 1
    assert _fuses(ok, normuon=True) == 0
    assert _fuses(ok, precision="fp32") == 0
    assert _fuses(ok, keep=True) == 0
    # 12 columns: rows are not 16-byte chunks
    assert _fuses(ok + [wl.ParamSpec("odd", (24, 12), "bf16")]) == 0
    # a weight whose rows start off 16-byte alignment
    assert _fuses(ok, offset=8) == 0
    assert L.lib().mo_plan_fuses_update(None) == 0
    assert L.lib().mo_plan_keep_ns_output(None, 1) == L.MO_EINVAL


def test_exclude_mask_validation():
    ok = dict(view=(2, 12, 8), split=(4, 8))
    for split, excl, want in (((4, 8), (1,), L.MO_OK), ((4, 8), (0, 1), L.MO_ESHAPE),
                              ((4, 8), (2,), L.MO_ESHAPE), (None, (0,), L.MO_ESHAPE)):
        kw = dict(ok, split=split)
        d = [api.make_desc("f", (24, 8), ident=1, exclude=excl, **kw)]
        arr = (L.ParamDesc * 1)(*d)
        out = (L.RouteOut * 1)()
        ng = C.c_int32()
        assert L.lib().mo_route(arr, 1, out, C.byref(ng)) == want, (split, excl)
        if want == L.MO_OK:
            assert (out[0].algorithm, out[0].nslices) == (L.MO_ALG_MUON, 2)
    # one identity, two registrations that disagree on the excluded pieces
    d = [api.make_desc("f", (24, 8), ident=1, exclude=(1,), **ok),
         api.make_desc("f2", (24, 8), ident=1, exclude=(0,), **ok)]
    arr = (L.ParamDesc * 2)(*d)
    out = (L.RouteOut * 2)()
    assert L.lib().mo_route(arr, 2, out, C.byref(C.c_int32())) == L.MO_ECONFLICT


def test_excluded_piece_alignment_and_buffers():
    """An excluded piece is an AdamW segment at the param's element offset:
    it needs exp_avg / exp_avg_sq and 16-byte aligned starts."""
    ok = wl.ParamSpec("f", (24, 8), "bf16", view=(2, 12, 8), split=(4, 8), exclude=(1,))
    h = C.c_void_p()
    hp = api.make_hparams()
    arr = _fake_entries([ok])
    L.check("plan", L.lib().mo_plan_create(arr, 1, C.byref(hp), None, C.byref(h)))
    assert L.lib().mo_plan_num_slices(h) == 2
    L.lib().mo_plan_destroy(h)
    arr = _fake_entries([ok])
    arr[0].exp_avg = None
    assert L.lib().mo_plan_create(arr, 1, C.byref(hp), None, C.byref(h)) == L.MO_EINVAL
    # rows of 6 bf16 columns: the excluded piece at row 3 starts 36 bytes in
    bad = wl.ParamSpec("f", (12, 6), "bf16", view=(2, 6, 6), split=(3, 3), exclude=(1,))
    arr = _fake_entries([bad])
    assert L.lib().mo_plan_create(arr, 1, C.byref(hp), None, C.byref(h)) == L.MO_EALIGN


def test_lr_schedule_matches_oracle():
    """mo_lr_at against the oracle's token-clock schedule over every phase,
    both peaks, and a shortened schedule; bad arguments are MO_EINVAL."""
    from oracle import schedule as osched
    taus = [0.0, 1.0, 1e6, 0.7e9, 1.999e9, 2e9, 50e9, 163.9e9, 164e9, 164e9 + 1,
            170e9, 185e9, 192.99e9, 193e9, 1e12]
    for peak in (0.01, 3e-4):
        for t in taus:
            assert api.lr_at(t, peak) == pytest.approx(osched.lr_at(t, peak), rel=1e-14, abs=0)
    short = dict(warmup=10.0, stable_end=40.0, end=100.0, floor=1e-4)
    for t in np.linspace(0, 120, 241):
        assert api.lr_at(t, 0.02, **short) == pytest.approx(osched.lr_at(t, 0.02, **short),
                                                            rel=1e-14, abs=0)
    c, oc = api.TokenClock(), osched.TokenClock()
    for w in [0.5e9] * 4 + [80e9, 82e9, 14.5e9, 14.5e9]:
        got, want = c.advance(w), oc.advance(w)
        assert got == pytest.approx(want, rel=1e-14)
    out = C.c_double()
    for bad in (L.LrSchedule(0.01, 5e9, 4e9, 193e9, 1e-5), L.LrSchedule(0.01, 2e9, 164e9, 193e9, 1.0)):
        assert L.lib().mo_lr_at(C.byref(bad), 1.0, C.byref(out)) == L.MO_EINVAL
    ok = L.LrSchedule(0.01, 2e9, 164e9, 193e9, 1e-5)
    assert L.lib().mo_lr_at(C.byref(ok), -1.0, C.byref(out)) == L.MO_EINVAL
    assert L.lib().mo_lr_at(C.byref(ok), float("nan"), C.byref(out)) == L.MO_EINVAL
    assert L.lib().mo_lr_at(None, 1.0, C.byref(out)) == L.MO_EINVAL


@pytest.mark.parametrize("table,rect,resident", [
    ([wl.CUBIC] * 5, True, True),          # gain 58: both
    ([wl.CUBIC] * 8, True, True),          # gain 657
    ([wl.CUBIC] * 9, False, False),        # gain 1478: past the threshold
    ([wl.QUINTIC] * 5, True, True),        # gain 537
    ([wl.QUINTIC] * 6, False, False),      # gain 1888
    ([wl.CUBIC, wl.QUINTIC, wl.CUBIC], True, True),
])
@pytest.mark.parametrize("gram_option", [True, False])
def test_gram_space_rule_host_only(table, rect, resident, gram_option):
    """Which slices run in Gram space (mo_plan_slice_algorithms): bf16,
    the table's gain prod a_k^2 <= 1024, then rectangular GEMM slices (any
    rows) and slice-resident slices with short side >= 64; square GEMM
    slices, short sides below 64 and the fp32 path never."""
    specs = (wl.ParamSpec("rect", (256, 640), "bf16"), wl.ParamSpec("square", (256, 256), "bf16"),
             wl.ParamSpec("resident", (128, 512), "bf16"), wl.ParamSpec("thin", (40, 512), "bf16"),
             wl.ParamSpec("rect32", (256, 640), "f32"))
    for precision in ("bf16", "fp32"):
        arr = _fake_entries(specs)
        hp = api.make_hparams(coeffs=table, ns_precision=precision)
        opts = api.plan_options(gram_space=gram_option)
        h = C.c_void_p()
        L.check("plan", L.lib().mo_plan_create(arr, len(specs), C.byref(hp), C.byref(opts),
                                               C.byref(h)))
        try:
            n = L.lib().mo_plan_num_slices(h)
            out = (C.c_int32 * n)()
            L.check("algos", L.lib().mo_plan_slice_algorithms(h, out, n))
            on = gram_option and precision == "bf16"
            want_gram = [on and rect, False, on and resident, False, on and rect]
            assert [bool(v & 1) for v in out] == want_gram
            kinds = [v >> 1 for v in out]
            if precision == "bf16":
                assert kinds == [0, 0, 2, 2, 0]
            else:
                assert kinds == [0, 0, 0, 0, 0]
            assert L.lib().mo_plan_gram_space(h) == int(any(want_gram))
        finally:
            L.lib().mo_plan_destroy(h)


def test_plan_entries_checked_before_the_library_sees_them():
    """api.Plan refuses a gradient or state whose dtype, size, layout or
    device does not match its parameter before calling mo_plan_create (the
    library reads G with W's dtype and every buffer with W's element count,
    so such an entry would read past an allocation).  CPU tensors only."""
    import torch
    spec = wl.ParamSpec("w", (8, 16), "bf16")
    desc = api.make_desc(spec.name, spec.shape)

    def entry(**over):
        e = {"desc": desc, "param": torch.zeros(8, 16, dtype=torch.bfloat16),
             "grad": torch.zeros(8, 16, dtype=torch.bfloat16),
             "momentum": torch.zeros(8, 16)}
        e.update(over)
        return e

    hp = api.make_hparams()
    bad = [(TypeError, dict(grad=torch.zeros(8, 16))),                          # fp32 grad
           (ValueError, dict(grad=torch.zeros(10, dtype=torch.bfloat16))),      # size
           (ValueError, dict(grad=torch.zeros(16, 8, dtype=torch.bfloat16).t())),  # layout
           (ValueError, dict(momentum=torch.zeros(8, 8))),                       # state size
           (TypeError, dict(momentum=torch.zeros(8, 16, dtype=torch.bfloat16))),
           (ValueError, dict(normuon_v=torch.zeros(16))),                         # rows
           (ValueError, dict(grad=torch.zeros(8, 16, dtype=torch.bfloat16, device="meta"))),
           (ValueError, dict(param=torch.zeros(4, 16, dtype=torch.bfloat16)))]
    for exc, over in bad:
        with pytest.raises(exc):
            api.Plan([entry(**over)], hp)


def _group(alg, specs, first, **hp):
    arr = _fake_entries(specs, normuon=hp.get("normuon", False))
    for i in range(len(specs)):
        arr[i].desc.ident = first + i
    g = L.Group()
    g.algorithm = L.MO_ALG_MUON if alg == "muon" else L.MO_ALG_ADAMW
    g.nparams = len(specs)
    g.params = C.cast(arr, C.POINTER(L.Param))
    g.hp = api.make_hparams(**hp)
    return g, arr


def test_group_table_host_only():
    """mo_plan_create_groups: plan order is group by group, routes report each
    group's algorithm and decay, slices come from each param's view; the
    table is validated before anything is built."""
    mat = wl.ParamSpec("q", (96, 96), "bf16")
    heads = wl.ParamSpec("h", (256, 64), "bf16", view=(2, 128, 64))
    emb = wl.ParamSpec("e", (64, 32), "bf16", wl.ROLE_EMBEDDING)
    gain = wl.ParamSpec("n", (32,), "bf16", wl.ROLE_NORM)
    keep = []
    gs = [_group("muon", [mat], 0, muon_lr=0.02, muon_wd=0.1),
          _group("muon", [heads], 10, muon_lr=0.005, coeffs=[wl.QUINTIC] * 5, normuon=True),
          _group("adamw", [emb], 20, adamw_lr=1e-3, adamw_wd=0.01),
          _group("adamw", [gain], 30, adamw_lr=3e-4, beta1=0.8)]
    keep += [a for _, a in gs]
    table = (L.Group * 4)(*[g for g, _ in gs])
    h = C.c_void_p()
    L.check("groups", L.lib().mo_plan_create_groups(table, 4, None, C.byref(h)))
    try:
        assert L.lib().mo_plan_num_groups(h) == 4 and L.lib().mo_plan_num_params(h) == 4
        out = (L.RouteOut * 4)()
        L.check("route", L.lib().mo_plan_route(h, out, 4))
        got = [(o.algorithm, o.decay, o.group, o.nslices) for o in out]
        assert got == [(L.MO_ALG_MUON, 1, 0, 1), (L.MO_ALG_MUON, 0, 1, 2),
                       (L.MO_ALG_ADAMW, 1, 2, 0), (L.MO_ALG_ADAMW, 0, 3, 0)]
        n = L.lib().mo_plan_num_slices(h)
        sl = (C.c_int64 * (4 * n))()
        L.check("slices", L.lib().mo_plan_slices(h, sl, n))
        assert [tuple(sl[4 * k:4 * k + 4]) for k in range(n)] == \
            [(0, 0, 96, 96), (1, 0, 128, 64), (1, 128, 128, 64)]
    finally:
        L.lib().mo_plan_destroy(h)

    def create(groups):
        t = (L.Group * len(groups))(*groups)
        hh = C.c_void_p()
        st = L.lib().mo_plan_create_groups(t, len(groups), None, C.byref(hh))
        if st == L.MO_OK:
            L.lib().mo_plan_destroy(hh)
        return st

    dup, a1 = _group("muon", [mat], 0)
    dup2, a2 = _group("adamw", [gain], 0)             # same identity 0
    assert create([dup, dup2]) == L.MO_ECONFLICT
    flat, a3 = _group("muon", [gain], 40)             # a 1-D param in a Muon group
    assert create([flat]) == L.MO_ESHAPE
    n1, a4 = _group("adamw", [emb], 50, max_norm=1.0)
    n2, a5 = _group("adamw", [gain], 60, max_norm=2.0)
    assert create([n1, n2]) == L.MO_EINVAL            # the clip norm is joint
    bad, a6 = _group("muon", [mat], 70)
    bad.algorithm = 7
    assert create([bad]) == L.MO_EINVAL
    frozen = api.make_desc("f", (8, 8), requires_grad=False, ident=80)
    arr = (L.Param * 1)()
    arr[0].desc = frozen
    g = L.Group()
    g.algorithm, g.nparams, g.params = L.MO_ALG_MUON, 1, C.cast(arr, C.POINTER(L.Param))
    g.hp = api.make_hparams()
    assert create([g]) == L.MO_EEMPTY


def test_noalloc_limits_refused_before_any_launch():
    """adamw_clip_step_noalloc: more than 64 items with a gradient, or more
    elements than its fixed scratch covers, is refused (MO_EWORKSPACE) on
    the host, before the device is touched (no GPU here)."""
    lib = L.lib()
    items = (L.AdamwItem * 65)()
    for i in range(65):
        items[i].param, items[i].grad = _fake_ptr(4 * i), _fake_ptr(4 * i + 1)
        items[i].exp_avg, items[i].exp_avg_sq = _fake_ptr(4 * i + 2), _fake_ptr(4 * i + 3)
        items[i].numel, items[i].dtype, items[i].step = 1024, L.MO_BF16, 1
    assert lib.adamw_clip_step_noalloc(items, 65, 1e-3, 0.9, 0.95, 1e-8, 1.0, None, None) == \
        L.MO_EWORKSPACE
    assert "64" in lib.mo_last_error().decode()
    items[0].numel = 130016 * 4 * 2048 + 1          # one block past the partial capacity
    assert lib.adamw_clip_step_noalloc(items, 1, 1e-3, 0.9, 0.95, 1e-8, 1.0, None, None) == \
        L.MO_EWORKSPACE
    items[0].numel, items[0].step = 1024, 0
    assert lib.adamw_clip_step_noalloc(items, 1, 1e-3, 0.9, 0.95, 1e-8, 1.0, None, None) == \
        L.MO_EINVAL
