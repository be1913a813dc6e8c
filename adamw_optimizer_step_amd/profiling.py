"""Hardware counters -> per-launch figures of the library's kernels.

rocprofv3 ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` report KiB per
dispatch.  Each counter is scaled by what it reads for k_diag_copy, a plain
copy of a known byte count run in the same process (``bench.py
--copy-calibration``): scale = known bytes / counted bytes.  ``--pmc
MfmaUtil`` gives the percentage of MFMA-busy cycles per dispatch.

One summary file covers one workload, coefficient set and NS precision, with
a section per kernel.  Each section records a digest of that kernel's
sources, so figures taken before the kernel changed are recognised as stale.

Command line (writes the summary to stdout)::

    python -m adamw_optimizer_step_amd.profiling counters \\
        --workload dense_decoder_1p2b --coeffs cubic --precision bf16 \\
        --copy-bytes N --fetch FETCH.csv --write WRITE.csv [--mfma MFMA.csv] \\
        --command "<the rocprofv3 commands, ;; separated>"
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import sys
from collections import defaultdict
from typing import Dict, List, Optional

_CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
# sources that define each measured kernel and its launch configuration
KERNEL_SOURCES = {
    "k_ns_gemm": ("ns.hip", "ns_host.cpp", "kernels.hpp", "common.hpp"),
    "k_ns_small": ("ns.hip", "ns_host.cpp", "kernels.hpp", "common.hpp"),
    "k_ns_prep": ("ns.hip", "ns_host.cpp", "kernels.hpp", "common.hpp"),
    "k_momentum": ("elementwise.hip", "kernels.hpp", "common.hpp"),
    "k_adam_sumsq": ("elementwise.hip", "kernels.hpp", "common.hpp"),
    "k_adam_apply": ("elementwise.hip", "kernels.hpp", "common.hpp"),
    "k_rows": ("elementwise.hip", "kernels.hpp", "common.hpp"),
}


def summary_name(workload: str, coeffs: str, precision: str) -> str:
    return f"counters_{workload}_{coeffs}_{precision}.md"


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(_CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _per_dispatch(path: str, counter: str) -> Dict[str, List[float]]:
    """kernel name -> counter value per dispatch, in dispatch order."""
    rows = defaultdict(list)
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") != counter:
                continue
            rows[r["Kernel_Name"]].append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    return {k: [v for _, v in sorted(d)] for k, d in rows.items()}


def _match(table: Dict[str, List[float]], kernel: str) -> List[float]:
    out: List[float] = []
    for name, vals in table.items():
        if re.search(r"(^|::|\s)" + re.escape(kernel) + r"(<|\()", name):
            out.extend(vals)
    return out


def counters_summary(workload: str, coeffs: str, precision: str, copy_bytes: int,
                     fetch_csv: str, write_csv: str,
                     mfma_csv: Optional[str] = None) -> Dict[str, object]:
    """Calibrated bytes per launch (and mean MfmaUtil) of every library kernel
    present in the counter files."""
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    mfma = _per_dispatch(mfma_csv, "MfmaUtil") if mfma_csv else {}
    cf, cw = _match(fetch, "k_diag_copy"), _match(write, "k_diag_copy")
    if not (cf and cw):
        raise SystemExit("counter files lack the k_diag_copy calibration")
    sf = copy_bytes / (1024.0 * sum(cf) / len(cf))
    sw = copy_bytes / (1024.0 * sum(cw) / len(cw))
    kernels: Dict[str, Dict[str, object]] = {}
    for k in KERNEL_SOURCES:
        kf, kw = _match(fetch, k), _match(write, k)
        if not (kf and kw):
            continue
        e: Dict[str, object] = {
            "source_digest": source_digest(k), "launches": len(kf),
            "fetch_bytes_per_launch": sf * 1024.0 * sum(kf) / len(kf),
            "write_bytes_per_launch": sw * 1024.0 * sum(kw) / len(kw),
        }
        m = _match(mfma, k)
        if m:
            e["mfma_util_pct"] = sum(m) / len(m)
        kernels[k] = e
    if not kernels:
        raise SystemExit("counter files hold none of the library's kernels")
    return {"workload": workload, "coeffs": coeffs, "precision": precision,
            "copy_bytes": copy_bytes, "scale_fetch": sf, "scale_write": sw,
            "kernels": kernels}


def _fmt(v) -> str:
    return f"{v:.6g}" if isinstance(v, float) else str(v)


def write_summary(s: Dict[str, object], commands: List[str], out=None) -> None:
    out = out if out is not None else sys.stdout

    def p(*a):
        print(*a, file=out)

    p(f"# Counter summary: {s['workload']} ({s['coeffs']}, {s['precision']})")
    p()
    p("Commands (one MI355X, repository root):")
    p()
    for c in commands:
        p("    " + c)
    p()
    p("Bytes are FETCH_SIZE and WRITE_SIZE per launch, each scaled by the ratio of the known")
    p("k_diag_copy size to what the counter reads for it; mfma_util_pct is MfmaUtil averaged")
    p("over the kernel's launches.")
    p()
    for k in ("workload", "coeffs", "precision", "copy_bytes", "scale_fetch", "scale_write"):
        p(f"{k}: {_fmt(s[k])}")
    for name, e in s["kernels"].items():
        p()
        p(f"[{name}]")
        for k, v in e.items():
            p(f"{k}: {_fmt(v)}")


def read_summary(path: str) -> Optional[Dict[str, object]]:
    """The summary as {key: value, ..., "kernels": {name: {key: value}}}, or
    None if the file does not exist."""
    if not os.path.exists(path):
        return None
    top: Dict[str, object] = {}
    kernels: Dict[str, Dict[str, str]] = {}
    cur: Optional[Dict[str, str]] = None
    with open(path) as f:
        for line in f:
            line = line.rstrip("\n")
            if line.startswith("    ") or line.startswith("#"):
                continue
            m = re.fullmatch(r"\[(\w+)\]", line.strip())
            if m:
                cur = kernels.setdefault(m.group(1), {})
                continue
            if ":" not in line:
                continue
            k, v = line.split(":", 1)
            (cur if cur is not None else top)[k.strip()] = v.strip()
    top["kernels"] = kernels
    return top


def kernel_figures(path: str, kernel: str, workload: str, coeffs: str,
                   precision: str) -> Optional[Dict[str, float]]:
    """The kernel's counted figures from the summary at `path`, or None when
    the summary is for another configuration, lacks the kernel, or predates
    the kernel's current sources."""
    s = read_summary(path)
    if not s or s.get("workload") != workload or s.get("coeffs") != coeffs or \
            s.get("precision") != precision:
        return None
    e = s["kernels"].get(kernel)
    if not e or e.get("source_digest") != source_digest(kernel):
        return None
    return {k: float(v) for k, v in e.items() if k != "source_digest"}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(prog="python -m adamw_optimizer_step_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("counters")
    t.add_argument("--workload", required=True)
    t.add_argument("--coeffs", default="cubic", choices=["cubic", "quintic"])
    t.add_argument("--precision", default="bf16", choices=["bf16", "fp32"])
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--mfma")
    t.add_argument("--command", default="")
    a = ap.parse_args(argv)
    s = counters_summary(a.workload, a.coeffs, a.precision, a.copy_bytes, a.fetch, a.write,
                         a.mfma)
    write_summary(s, [c.strip() for c in a.command.split(";;") if c.strip()])
    return 0


if __name__ == "__main__":
    sys.exit(main())
