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


# Gram space: shortest short side in the slice-resident kernel
GS_MIN_SHORT = 64


def ns_work(slices, coeffs, elem, w_elem=None, gram_space=False, sxs_on_chip=False):
    """Newton-Schulz work per step, from the per-slice unit figures (s = short
    side, l = long side of each slice, N iterations):
    * dense flops, the method's count: 4 s^2 l per iteration (A = X X^T and
      P X), + 2 s^3 for a quintic-type row;
    * executed flops, plain iteration with the symmetric Gram: 3 s^2 l
      (+ s^3) per iteration; Gram-space sequence (cubic rows): s^2 l for
      A0 = X0 X0^T, 3 N - 3 symmetric s x s products of s^3 each, and
      2 s^2 l for X_N = Q_N X0.  With ``gram_space`` set, a slice runs in
      Gram space under the library's rule: in the slice-resident kernel
      (sxs_on_chip) when s >= 64, in the GEMM path when 4 l >= 5 s (a square
      slice executes the same flops either way and stays plain);
    * HBM bytes when X does not stay on chip: plain, one read of X0 for the
      first Gram, then a read of X and a write of X' per iteration:
      elem * s * l * (2 N + 1); Gram space, two reads of X0 and one write of
      X_N, elem * s * l * 3, plus per s x s product two operands, the E term
      and the result, 4 elem s^2, and A0 and Q1, 2 elem s^2 (none when the
      s x s matrices stay in LDS, sxs_on_chip).  With the Muon
      update fused into the last launch (w_elem = weight element size) the
      last write is replaced by a read and a write of W: + (2 w_elem - elem) s l.
    Returns (dense_flops, executed_flops, bytes)."""
    dense = exe = byt = 0.0
    n = len(coeffs)
    for r, c in slices:
        s, l = float(min(r, c)), float(max(r, c))
        for a, b, cc in coeffs:
            dense += 4.0 * s * s * l
            if cc != 0.0:
                dense += 2.0 * s ** 3
        gs = gram_space and (s >= GS_MIN_SHORT if sxs_on_chip else 4 * l >= 5 * s)
        if gs:
            exe += 3.0 * s * s * l + (3 * n - 3) * s ** 3
            byt += elem * s * l * 3
            if not sxs_on_chip:
                byt += (4 * (3 * n - 3) + 2) * elem * s * s
        else:
            for a, b, cc in coeffs:
                exe += 3.0 * s * s * l + (s ** 3 if cc != 0.0 else 0.0)
            byt += elem * s * l * (2 * n + 1)
        if w_elem is not None:
            byt += (2 * w_elem - elem) * s * l
    return dense, exe, byt


# slices whose padded short side is 128 run in the slice-resident kernel (bf16)
SMALL_SIDE = 128


def build_plan(w, coeffs, precision, normuon):
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
    hp = api.make_hparams(coeffs=coeffs, ns_precision=precision, normuon=normuon)
    plan = api.Plan(ents, hp)
    return plan, ents, routes


def cpu_baseline(w, coeffs, normuon, budget_s: float):
    """The fp64 oracle on a bounded sample of the same workload, extrapolated
    to one full step: one Muon matrix of each distinct shape and a contiguous
    slab of the AdamW elements."""
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
    t_total = 0.0
    parts = []
    spent = 0.0
    for key, (idx, count) in shapes.items():
        p = w.params[idx]
        G = wl.from_storage(wl.grad(w, idx, 1), p.dtype).astype(np.float64)
        W = wl.from_storage(wl.init_weight(w, idx), p.dtype).astype(np.float64)
        t0 = time.perf_counter()
        omuon.muon_param_step(W, G, np.zeros_like(G), expand(p.shape, p.view, p.split), coeffs,
                              0.01, 0.95,
                              normuon_v=np.zeros(p.shape[0]) if normuon else None)
        dt = time.perf_counter() - t0
        spent += dt
        t_total += dt * count
        parts.append(f"{count}x{p.shape}")
        if spent > budget_s:
            break
    n_adam = 0
    if adam_elems:
        n = min(adam_elems, 1 << 22)
        g = wl.draw_f32(w.seed, 1, 0, (n,), w.grad_std).astype(np.float64)
        W = wl.draw_f32(w.seed, 0, 0, (n,), w.init_std).astype(np.float64)
        t0 = time.perf_counter()
        T = oadamw.global_norm([g])
        oadamw.adamw_update(W, g, np.zeros(n), np.zeros(n), 1, 3e-4, 0.9, 0.95, 1e-8, 0.0,
                            oadamw.clip_factor(T, 1.0))
        dt = time.perf_counter() - t0
        t_total += dt * adam_elems / n
        n_adam = n
    return {"value": 1.0 / t_total, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": (f"fp64 numpy oracle: one full Muon step of one matrix per distinct "
                       f"slice shape (weighted by count: {', '.join(parts)}) and AdamW on "
                       f"{n_adam} of {adam_elems} elements, extrapolated to one full step; "
                       f"{spent:.1f}s of Muon work measured")}


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
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dense_decoder_1p2b")
    ap.add_argument("--coeffs", default="cubic", choices=["cubic", "quintic"])
    ap.add_argument("--precision", default="bf16", choices=["bf16", "fp32"])
    ap.add_argument("--timing-steps", type=int, default=3)
    ap.add_argument("--separate-update", action="store_true",
                    help="keep O and apply the Muon update in its own row pass instead of "
                         "inside the last Newton-Schulz launch")
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
    plan, ents, routes = build_plan(w, coeffs, args.precision, w.normuon)
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
    t0 = time.perf_counter()
    for _ in range(args.steps):
        plan.step(workspace=ws)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    log(f"{ms_per_step:.3f} ms/step")

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

    # algorithmic work
    fused = plan.fuses_update()
    gspace = plan.gram_space()
    welt = w.params[0].dtype == "bf16" and 2 or 4
    slices = [(r, c) for _, _, r, c in plan.slices()]
    elem = 2 if args.precision == "bf16" else 4
    muon_elems = sum(r * c for r, c in slices)
    adam_elems = sum(p.numel for p, r in zip(w.params, routes) if r[0] == L.MO_ALG_ADAMW)
    small = [sc for sc in slices if args.precision == "bf16" and min(sc) <= SMALL_SIDE]
    large = [sc for sc in slices if not (args.precision == "bf16" and min(sc) <= SMALL_SIDE)]
    peak = BF16_PEAK_TFLOPS if args.precision == "bf16" else FP32_PEAK_TFLOPS
    # the dominant Newton-Schulz kernel and the slices it processes
    cands = [(name, part) for name, part in (("ns_gemm", large), ("ns_small", small))
             if name in kern and part]
    roofline = None
    if cands:
        kname, part = max(cands, key=lambda x: kern[x[0]]["ms_per_step"])
        g = kern[kname]
        dense, exe, nbytes = ns_work(part, coeffs, elem, welt if fused else None,
                                     gram_space=gspace, sxs_on_chip=kname == "ns_small")
        n = g["launches_per_step"]
        t = g["avg_launch_ms"] * 1e-3
        # the binding roof is the one with the longer ideal time: for the
        # GEMM launches on the method's dense count, for the slice-resident
        # kernel on the flops it executes (in Gram space its s x s work is
        # small next to its passes over X)
        flops = dense if kname == "ns_gemm" else exe
        mfma_bound = flops / (peak * 1e12) >= nbytes / (HBM_PEAK_GBS * 1e9)
        if mfma_bound:
            achieved = dense / n / t / 1e12
            roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                        "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
        else:
            achieved = nbytes / n / t / 1e9
            roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
        roofline.update({
            "traffic": None, "kernel": "k_" + kname, "avg_launch_ms": g["avg_launch_ms"],
            "launches_per_step": n, "slices": len(part),
            "dense_flops_per_launch": dense / n, "dense_tflops": round(dense / n / t / 1e12, 2),
            "executed_tflops": round(exe / n / t / 1e12, 2),
            "algorithmic_bytes_per_launch": nbytes / n,
            "algorithmic_gbs": round(nbytes / n / t / 1e9, 1),
            "executed_frac": round(exe / n / t / 1e12 / peak, 4),
            "symmetry_exploited": kname == "ns_gemm",
            "algorithm": "gram_space" if gspace else "plain"})
    hbm = {}
    elt = w.params[0].dtype == "bf16" and 2 or 4
    if "momentum" in kern:
        b = muon_elems * (elt + 4 + 4 + elt)
        hbm["momentum"] = round(b / (kern["momentum"]["ms_per_step"] * 1e-3) / 1e9, 1)
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
    cnt = {k: counted(k, w.key, args.coeffs, args.precision)
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
        cpu = cpu_baseline(w, coeffs, w.normuon, args.cpu_budget)

    value = 1e3 / ms_per_step
    out = {
        "metric": METRIC, "value": round(value, 4), "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": args.precision, "data": "synthetic",
        "config": {"workload": w.key, "muon_params": muon_elems, "adamw_params": adam_elems,
                   "muon_slices": len(slices), "ns_steps": len(coeffs), "coeffs": args.coeffs,
                   "ns_precision": args.precision, "normuon": bool(w.normuon),
                   "fused_update": fused, "gram_space": gspace,
                   "param_dtype": w.params[0].dtype, "state_dtype": "f32"},
        "roofline": roofline,
        "ns_dense_tflops_pct_of_peak": (round(100 * roofline["dense_tflops"] / peak, 2)
                                        if roofline else None),
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
