"""Benchmark: hybrid Muon + AdamW optimizer steps/s on one MI355X.

Default workload: the dense decoder parameter set (d=2048, 24 layers, SwiGLU
I=5632; 1.233B Muon params in 168 matrices, 262.8M AdamW params in a tied
128256x2048 embedding and 49 RMSNorm gains), bf16 params and grads N(0,1e-3),
fp32 optimizer states, 5 cubic Newton-Schulz iterations in bf16 with fp32
accumulation.  One step = one full hybrid step (momentum, Newton-Schulz,
update for every Muon matrix; clip + AdamW for every AdamW parameter) through
``mo_grouped_step``.  Inputs are resident in HBM before timing starts.

Prints one JSON line (rank 0, N=1) with the steps/s, a roofline entry for the
dominant kernel (the batched Newton-Schulz GEMM, from HIP events on its own
stream, in extra steps that run every kernel alone), and the fp64 oracle
timed on a bounded sample on the host cores.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Muon+AdamW optimizer steps/sec at 1.24B params; NS MFMA util %; AdamW HBM GB/s"
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3    # MI355X fp32 matrix
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def workload_by_name(name: str, coeffs: str = "cubic"):
    import workloads as wl
    table = {
        "dense_decoder_1p2b": lambda: wl.dense_decoder(),
        "dense_decoder_1p2b_fused_normuon": lambda: wl.dense_decoder(fused_gate_up=True,
                                                                     normuon=True),
        "head_batched_mla_kda": lambda: wl.head_batched(),
        "ns_sweep_1024x1024": lambda: wl.ns_sweep(1024, 1024, coeffs),
        "ns_sweep_4096x1024": lambda: wl.ns_sweep(4096, 1024, coeffs),
    }
    return table[name]()


def ns_work(slices, coeffs, elem, w_elem=None):
    """Newton-Schulz work per step from the per-slice unit figures.

    ``slices``: (rows, cols, gram_space, kernel) per slice, kernel one of
    'gemm128', 'gemm256', 'resident' (the library's own choice, from
    mo_plan_slice_algorithms).  With s the short side, l the long side and N
    the table's rows:
    * method flops, the method's own work with the symmetric Gram: 3 s^2 l
      per iteration (s^2 l for A = X X^T, 2 s^2 l for P X), + s^3 for a
      quintic-type row (A^2);
    * dense flops, the same without symmetry: 4 s^2 l (+ 2 s^3);
    * executed flops, what the kernels run: the plain iteration executes the
      method flops; the Gram-space sequence executes s^2 l for A0 = X0 X0^T,
      3 N - 3 symmetric s x s products of s^3 each (+ one more per
      quintic-type row, in the slice-resident kernel) and 2 s^2 l for
      X_N = Q_N X0;
    * HBM bytes of the iterate traffic: plain, one read of X0 for the first
      Gram, then a read of X and a write of X' per iteration,
      elem s l (2 N + 1); Gram space, two reads of X0 and one write of X_N,
      3 elem s l, plus for the GEMM kernels per s x s product two operands,
      the E term and the result (4 elem s^2) and A0 and Q1 (2 elem s^2).  With
      the Muon update fused into the last launch (w_elem = weight element
      size) the last write becomes a read and a write of W:
      + (2 w_elem - elem) s l.
    Returns a dict of totals."""
    t = {"method": 0.0, "dense": 0.0, "executed": 0.0, "bytes": 0.0}
    n = len(coeffs)
    nq = sum(1 for _, _, cc in coeffs if cc != 0.0)
    for r, c, gram, kernel in slices:
        s, l = float(min(r, c)), float(max(r, c))
        t["method"] += n * 3.0 * s * s * l + nq * s ** 3
        t["dense"] += n * 4.0 * s * s * l + nq * 2.0 * s ** 3
        if gram:
            prods = 3 * n - 3 + (nq if kernel == "resident" else 0)
            t["executed"] += 3.0 * s * s * l + prods * s ** 3
            t["bytes"] += elem * s * l * 3
            if kernel != "resident":
                t["bytes"] += (4 * (3 * n - 3) + 2) * elem * s * s
        else:
            t["executed"] += n * 3.0 * s * s * l + nq * s ** 3
            t["bytes"] += elem * s * l * (2 * n + 1)
        if w_elem is not None:
            t["bytes"] += (2 * w_elem - elem) * s * l
    return t


def build_plan(w, coeffs, precision, normuon, spectral_cap=0.0, spectral_iters=8):
    import torch

    import workloads as wl
    from adamw_optimizer_step_amd import _lib as L
    from adamw_optimizer_step_amd import api

    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    descs = [api.make_desc(p.name, p.shape, p.role, p.no_decay, True, i, p.view, p.split)
             for i, p in enumerate(w.params)]
    routes, _ = api.route(descs)
    ents = []
    for i, (p, r) in enumerate(zip(w.params, routes)):
        e = {"desc": descs[i],
             "param": wl.draw_device(w.seed, 0, i, p.shape, w.init_std, p.dtype),
             "grad": wl.draw_device(w.seed, 1, i, p.shape, w.grad_std, p.dtype)}
        assert e["param"].dtype == tdt[p.dtype]
        if r[0] == L.MO_ALG_MUON:
            e["momentum"] = torch.zeros(p.shape, dtype=torch.float32, device="cuda")
            if normuon:
                e["normuon_v"] = torch.zeros(p.shape[0], dtype=torch.float32, device="cuda")
        elif r[0] == L.MO_ALG_ADAMW:
            e["exp_avg"] = torch.zeros(p.shape, dtype=torch.float32, device="cuda")
            e["exp_avg_sq"] = torch.zeros(p.shape, dtype=torch.float32, device="cuda")
        ents.append(e)
    hp = api.make_hparams(coeffs=coeffs, ns_precision=precision, normuon=normuon,
                          spectral_cap=spectral_cap, spectral_iters=spectral_iters)
    plan = api.Plan(ents, hp)
    return plan, ents, routes


def cpu_baseline(w, coeffs, normuon, budget_s: float, spectral_cap=0.0, spectral_iters=8):
    """The fp64 oracle on a bounded sample of the same workload, extrapolated
    to one full step: one Muon matrix of each distinct slice shape and a
    contiguous slab of the AdamW elements, timed in rounds over all shapes
    until about ``budget_s`` seconds of oracle work are spent (at least one
    round); each shape's time is its mean over the rounds."""
    import numpy as np

    import workloads as wl
    from oracle import adamw as oadamw
    from oracle import muon as omuon
    from oracle.views import expand
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = len(os.sched_getaffinity(0))
    shapes = {}
    adam_elems = 0
    for i, p in enumerate(w.params):
        if len(p.shape) == 2 and p.role == "matrix":
            key = tuple(tuple(sorted((r, c))) for _, r, c in expand(p.shape, p.view, p.split))
            shapes.setdefault(key, [i, 0])[1] += 1
        else:
            adam_elems += p.numel
    inputs = []
    for key, (idx, count) in shapes.items():
        p = w.params[idx]
        G = wl.from_storage(wl.grad(w, idx, 1), p.dtype).astype(np.float64)
        W = wl.from_storage(wl.init_weight(w, idx), p.dtype).astype(np.float64)
        inputs.append((p, G, W, count))
    n_adam = min(adam_elems, 1 << 22)
    if n_adam:
        ga = wl.draw_f32(w.seed, 1, 0, (n_adam,), w.grad_std).astype(np.float64)
        wa = wl.draw_f32(w.seed, 0, 0, (n_adam,), w.init_std).astype(np.float64)
    muon_s = [0.0] * len(inputs)
    adam_s = 0.0
    spent = 0.0
    rounds = 0
    while rounds == 0 or spent < budget_s:
        for j, (p, G, W, _) in enumerate(inputs):
            Wr, Br = W.copy(), np.zeros_like(G)
            t0 = time.perf_counter()
            omuon.muon_param_step(Wr, G, Br, expand(p.shape, p.view, p.split),
                                  coeffs, 0.01, 0.95,
                                  normuon_v=np.zeros(p.shape[0]) if normuon else None,
                                  spectral_cap_value=spectral_cap, spectral_iters=spectral_iters)
            dt = time.perf_counter() - t0
            muon_s[j] += dt
            spent += dt
        if n_adam:
            Wr, m0, v0 = wa.copy(), np.zeros(n_adam), np.zeros(n_adam)
            t0 = time.perf_counter()
            T = oadamw.global_norm([ga])
            oadamw.adamw_update(Wr, ga, m0, v0, 1, 3e-4, 0.9, 0.95, 1e-8, 0.0,
                                oadamw.clip_factor(T, 1.0))
            dt = time.perf_counter() - t0
            adam_s += dt
            spent += dt
        rounds += 1
    t_total = sum(m / rounds * count for m, (_, _, _, count) in zip(muon_s, inputs))
    if n_adam:
        t_total += adam_s / rounds * adam_elems / n_adam
    parts = [f"{count}x{p.shape}" for p, _, _, count in inputs]
    return {"value": 1.0 / t_total, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": (f"fp64 numpy oracle: one full Muon step of one matrix per distinct "
                       f"slice shape (weighted by count: {', '.join(parts)}) and AdamW on "
                       f"{n_adam} of {adam_elems} elements, extrapolated to one full step; "
                       f"{rounds} rounds, {spent:.1f}s of oracle work measured")}


def counted(kernel: str, workload: str, coeffs: str, precision: str):
    """The kernel's counter figures (calibrated HBM bytes per launch, mean
    MfmaUtil) from the committed summary for this workload, coefficient set
    and NS precision, or None when there is none or the kernel's sources have
    changed since the counters were taken."""
    from adamw_optimizer_step_amd import profiling
    path = os.path.join(ROOT, "profiles", profiling.summary_name(workload, coeffs, precision))
    return profiling.kernel_figures(path, kernel, workload, coeffs, precision)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dense_decoder_1p2b")
    ap.add_argument("--coeffs", default="cubic", choices=["cubic", "quintic"])
    ap.add_argument("--precision", default="bf16", choices=["bf16", "fp32"])
    ap.add_argument("--timing-steps", type=int, default=3)
    ap.add_argument("--separate-update", action="store_true",
                    help="keep O and apply the Muon update in its own row pass instead of "
                         "inside the last Newton-Schulz launch")
    ap.add_argument("--spectral-cap", type=float, default=0.0, metavar="TAU",
                    help="turn on the spectral-cap guard on the Muon buffer at cap TAU "
                         "(0 = off, the default)")
    ap.add_argument("--spectral-iters", type=int, default=8,
                    help="power iterations of the guard's estimate")
    ap.add_argument("--cpu-budget", type=float, default=20.0,
                    help="seconds of oracle work for the cpu_baseline sample (0 = skip)")
    ap.add_argument("--copy-calibration", type=int, default=1024, metavar="MIB",
                    help="size of the plain device copy (k_diag_copy) that calibrates "
                         "byte counters and gives the copy bandwidth (0 = skip)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this library runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        log("multi-GPU runs are not implemented: the sharding design is documented "
            "but only the one-GPU path exists")
        return 2

    import torch

    import workloads as wl
    from adamw_optimizer_step_amd import _lib as L

    if not torch.cuda.is_available():
        log("no HIP device visible")
        return 1
    torch.cuda.set_device(0)
    w = workload_by_name(args.workload, args.coeffs)
    coeffs = wl.coeff_table(args.coeffs, w.ns_steps)
    log(f"building {w.key} on {torch.cuda.get_device_name(0)}")
    plan, ents, routes = build_plan(w, coeffs, args.precision, w.normuon, args.spectral_cap,
                                    args.spectral_iters)
    if args.separate_update:
        plan.keep_ns_output(True)
    ws = plan.workspace(torch.device("cuda"))
    torch.cuda.synchronize()
    log(f"plan ready: {plan.workspace_bytes / 2**30:.2f} GiB workspace, "
        f"{len(plan.slices())} Muon slices")

    for _ in range(args.warmup):
        plan.step(workspace=ws)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done; timing {args.steps} steps")
    # each step bracketed by events on the launch stream (the step joins its
    # side stream back into it); the whole timed region by synchronisations
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    evs[0].record()
    for k in range(args.steps):
        plan.step(workspace=ws)
        evs[k + 1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per_step = sorted(evs[k].elapsed_time(evs[k + 1]) for k in range(args.steps))
    mid = len(per_step) // 2
    median_ms = per_step[mid] if len(per_step) % 2 else 0.5 * (per_step[mid - 1] + per_step[mid])
    mean_ms = 1e3 * elapsed / args.steps
    log(f"median {median_ms:.3f} ms/step, mean {mean_ms:.3f} ms/step (wall clock)")

    # per-kernel-class durations with HIP events on the launch stream; while
    # timing is on, the grouped step runs every kernel in order on one stream
    # (no AdamW overlap), so each duration is one kernel running alone
    lib = L.lib()
    L.check("timing", lib.mo_timing_enable(1))
    for _ in range(args.timing_steps):
        plan.step(workspace=ws)
    torch.cuda.synchronize()
    import ctypes as C
    kern = {}
    for k, name in enumerate(L.KERNEL_CLASSES):
        tot, n = C.c_double(0.0), C.c_int64(0)
        L.check("timing", lib.mo_timing_read(k, C.byref(tot), C.byref(n)))
        if n.value:
            kern[name] = {"ms_per_step": tot.value / args.timing_steps,
                          "launches_per_step": n.value / args.timing_steps,
                          "avg_launch_ms": tot.value / n.value}
    L.check("timing", lib.mo_timing_enable(0))

    # algorithmic work, per slice as the library runs it
    fused = plan.fuses_update()
    gspace = plan.gram_space()
    welt = w.params[0].dtype == "bf16" and 2 or 4
    algos = plan.slice_algorithms()
    slices = [(r, c) for _, _, r, c in plan.slices()]
    elem = 2 if args.precision == "bf16" else 4
    muon_elems = sum(r * c for r, c in slices)
    adam_elems = sum(p.numel for p, r in zip(w.params, routes) if r[0] == L.MO_ALG_ADAMW)
    by_kernel = {"ns_gemm": [], "ns_small": []}
    for (r, c), al in zip(slices, algos):
        if al is not None:
            by_kernel["ns_small" if al[1] == "resident" else "ns_gemm"].append((r, c) + al)
    peak = BF16_PEAK_TFLOPS if args.precision == "bf16" else FP32_PEAK_TFLOPS
    # the dominant Newton-Schulz kernel and the slices it processes
    cands = [(name, part) for name, part in by_kernel.items() if name in kern and part]
    roofline = None
    if cands:
        kname, part = max(cands, key=lambda x: kern[x[0]]["ms_per_step"])
        g = kern[kname]
        work = ns_work(part, coeffs, elem, welt if fused else None)
        n = g["launches_per_step"]
        t = g["avg_launch_ms"] * 1e-3
        # the binding roof is the one with the longer ideal time: for the
        # GEMM launches on the method's flops, for the slice-resident kernel
        # on the flops it executes (in Gram space its s x s work is small
        # next to its passes over X)
        flops = work["method"] if kname == "ns_gemm" else work["executed"]
        mfma_bound = flops / (peak * 1e12) >= work["bytes"] / (HBM_PEAK_GBS * 1e9)
        if mfma_bound:
            achieved = work["method"] / n / t / 1e12
            roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                        "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
        else:
            achieved = work["bytes"] / n / t / 1e9
            roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
        roofline.update({
            "traffic": None, "kernel": "k_" + kname, "avg_launch_ms": g["avg_launch_ms"],
            "launches_per_step": n, "slices": len(part),
            "method_flops_per_launch": work["method"] / n,
            "method_tflops": round(work["method"] / n / t / 1e12, 2),
            "dense_count_tflops": round(work["dense"] / n / t / 1e12, 2),
            "executed_tflops": round(work["executed"] / n / t / 1e12, 2),
            "executed_frac": round(work["executed"] / n / t / 1e12 / peak, 4),
            "algorithmic_bytes_per_launch": work["bytes"] / n,
            "algorithmic_gbs": round(work["bytes"] / n / t / 1e9, 1),
            "gram_space_slices": sum(1 for x in part if x[2]),
            "algorithm": "gram_space" if any(x[2] for x in part) else "plain"})
    hbm = {}
    elt = w.params[0].dtype == "bf16" and 2 or 4
    if "momentum" in kern:
        # with the guard on, two passes: B <- mu B + G, then D (and B <- kappa B
        # where the cap binds, not counted here)
        b = muon_elems * ((elt + 4 + 4 + elt) if args.spectral_cap <= 0
                          else (elt + 4 + 4) + (elt + 4 + elt))
        hbm["momentum"] = round(b / (kern["momentum"]["ms_per_step"] * 1e-3) / 1e9, 1)
    if "spectral" in kern:
        # the power iteration reads the fp32 buffer twice per iteration and
        # once more for the estimate
        b = muon_elems * 4 * (2 * args.spectral_iters + 1)
        hbm["spectral"] = round(b / (kern["spectral"]["ms_per_step"] * 1e-3) / 1e9, 1)
    if "adam_apply" in kern:
        t = sum(kern[k]["ms_per_step"] for k in ("adam_sumsq", "adam_norm", "adam_apply")
                if k in kern)
        hbm["adamw"] = round(adam_elems * (2 * elt + 16 + 2 * elt) / (t * 1e-3) / 1e9, 1)
    if "rows" in kern:
        hbm["update"] = round(muon_elems * (3 * elt) / (kern["rows"]["ms_per_step"] * 1e-3) / 1e9,
                              1)

    # plain copy of known size: counter calibration and practical HBM ceiling
    copy_gbs = None
    if args.copy_calibration > 0:
        nbytes = args.copy_calibration << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(7)
        dst = torch.empty_like(src)
        stream = torch.cuda.current_stream().cuda_stream
        L.check("mo_diag_copy", lib.mo_diag_copy(C.c_void_p(src.data_ptr()),
                                                 C.c_void_p(dst.data_ptr()), nbytes,
                                                 C.c_void_p(stream)))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        L.check("mo_diag_copy", lib.mo_diag_copy(C.c_void_p(src.data_ptr()),
                                                 C.c_void_p(dst.data_ptr()), nbytes,
                                                 C.c_void_p(stream)))
        e1.record()
        torch.cuda.synchronize()
        copy_gbs = round(2 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
        hbm["copy"] = copy_gbs
        del src, dst

    # counter-based figures (committed rocprofv3 summaries; null when stale)
    # (the summaries are of the default step: none applies with the guard on)
    cnt = {k: counted(k, w.key, args.coeffs, args.precision) if args.spectral_cap <= 0 else None
           for k in ("k_ns_gemm", "k_ns_small", "k_momentum", "k_rows", "k_adam_sumsq",
                     "k_adam_apply")}
    if roofline is not None:
        c = cnt.get(roofline["kernel"])
        roofline["traffic"] = (c["fetch_bytes_per_launch"] + c["write_bytes_per_launch"]
                               if c else None)
        roofline["mfma_util_pct"] = round(c["mfma_util_pct"], 2) \
            if c and "mfma_util_pct" in c else None
    hbm_counted = {}
    for name, ks in (("momentum", ("k_momentum",)), ("update", ("k_rows",)),
                     ("adamw", ("k_adam_sumsq", "k_adam_apply"))):
        cs = [cnt.get(k) for k in ks]
        t = sum(kern[n]["ms_per_step"] for n in kern
                if "k_" + n in ks or (name == "adamw" and n == "adam_norm"))
        if all(cs) and t > 0:
            b = sum((c["fetch_bytes_per_launch"] + c["write_bytes_per_launch"]) for c in cs)
            hbm_counted[name] = round(b / (t * 1e-3) / 1e9, 1)
        else:
            hbm_counted[name] = None

    cpu = None
    if args.cpu_budget > 0:
        log("timing the fp64 oracle on a bounded sample")
        cpu = cpu_baseline(w, coeffs, w.normuon, args.cpu_budget, args.spectral_cap,
                           args.spectral_iters)

    value = 1e3 / median_ms
    out = {
        "metric": METRIC, "value": round(value, 4), "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(median_ms, 4),
        "timing": "median of per-step HIP-event times on the launch stream",
        "mean_ms_per_step": round(mean_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": args.precision, "data": "synthetic",
        "config": {"workload": w.key, "muon_params": muon_elems, "adamw_params": adam_elems,
                   "muon_slices": len(slices), "ns_steps": len(coeffs), "coeffs": args.coeffs,
                   "ns_precision": args.precision, "normuon": bool(w.normuon),
                   "fused_update": fused, "gram_space": gspace,
                   "spectral_cap": args.spectral_cap if args.spectral_cap > 0 else None,
                   "param_dtype": w.params[0].dtype, "state_dtype": "f32"},
        "roofline": roofline,
        "ns_mfma_util_pct": roofline.get("mfma_util_pct") if roofline else None,
        "adamw_hbm_gbs": hbm.get("adamw"),
        "hbm_gbs": hbm,
        "hbm_gbs_counted": hbm_counted,
        "kernels": kern,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
