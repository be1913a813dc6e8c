"""Hardware byte counters -> per-launch HBM traffic of a kernel.

rocprofv3 ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` report KiB per
dispatch.  Each counter is scaled by what it reads for k_diag_copy, a plain
copy of a known byte count run in the same process (``bench.py
--copy-calibration``): scale = known bytes / counted bytes.  The summary
records a digest of the kernel sources, so a summary taken before the kernel
changed is recognised as stale.

Command line (writes a text summary to stdout)::

    python -m adamw_optimizer_step_amd.profiling traffic --kernel k_ns_gemm \\
        --workload dense_decoder_1p2b --copy-bytes N \\
        --fetch FETCH_counter_collection.csv --write WRITE_counter_collection.csv \\
        --command "<the rocprofv3 commands>"
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
    "k_momentum": ("elementwise.hip", "kernels.hpp", "common.hpp"),
    "k_adam_apply": ("elementwise.hip", "kernels.hpp", "common.hpp"),
    "k_rows": ("elementwise.hip", "kernels.hpp", "common.hpp"),
}


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(_CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _per_dispatch(path: str, counter: str) -> Dict[str, List[float]]:
    """kernel name -> counter value (bytes) per dispatch, in dispatch order."""
    rows = defaultdict(list)
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") != counter:
                continue
            rows[r["Kernel_Name"]].append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    return {k: [v * 1024.0 for _, v in sorted(d)] for k, d in rows.items()}


def _match(table: Dict[str, List[float]], kernel: str) -> List[float]:
    out: List[float] = []
    for name, vals in table.items():
        if re.search(r"(^|::|\s)" + re.escape(kernel) + r"(<|\()", name):
            out.extend(vals)
    return out


def traffic_summary(kernel: str, workload: str, copy_bytes: int, fetch_csv: str,
                    write_csv: str, coeffs: str = "cubic",
                    precision: str = "bf16") -> Dict[str, float]:
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    cf, cw = _match(fetch, "k_diag_copy"), _match(write, "k_diag_copy")
    kf, kw = _match(fetch, kernel), _match(write, kernel)
    if not (cf and cw and kf and kw):
        raise SystemExit("counter files lack the copy calibration or the kernel")
    sf = copy_bytes / (sum(cf) / len(cf))
    sw = copy_bytes / (sum(cw) / len(cw))
    return {
        "kernel": kernel, "workload": workload, "coeffs": coeffs, "precision": precision,
        "source_digest": source_digest(kernel),
        "launches": len(kf), "copy_bytes": copy_bytes,
        "copy_fetch_counted": sum(cf) / len(cf), "copy_write_counted": sum(cw) / len(cw),
        "scale_fetch": sf, "scale_write": sw,
        "fetch_bytes_per_launch": sf * sum(kf) / len(kf),
        "write_bytes_per_launch": sw * sum(kw) / len(kw),
    }


def read_summary(path: str) -> Optional[Dict[str, str]]:
    """The key: value lines of a summary file (None if absent)."""
    if not os.path.exists(path):
        return None
    out = {}
    with open(path) as f:
        for line in f:
            if line.startswith("    ") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(prog="python -m adamw_optimizer_step_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--kernel", required=True, choices=sorted(KERNEL_SOURCES))
    t.add_argument("--workload", required=True)
    t.add_argument("--coeffs", default="cubic", choices=["cubic", "quintic"])
    t.add_argument("--precision", default="bf16", choices=["bf16", "fp32"])
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--command", default="")
    a = ap.parse_args(argv)
    s = traffic_summary(a.kernel, a.workload, a.copy_bytes, a.fetch, a.write, a.coeffs,
                        a.precision)
    print(f"# HBM traffic of {a.kernel}, workload {a.workload} ({a.coeffs}, {a.precision})")
    print()
    print("Commands (one MI355X, repository root):")
    print()
    for c in a.command.split(";;"):
        if c.strip():
            print("    " + c.strip())
    print()
    for k, v in s.items():
        print(f"{k}: {v:.6g}" if isinstance(v, float) else f"{k}: {v}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
