"""bench.py's host-side contract: the one-GPU limit and the workload table
(no GPU is touched)."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_sweep_workload_names_carry_the_coefficients():
    assert bench.workload_by_name("ns_sweep_1024x1024", "quintic").key == \
        "ns_sweep_1024x1024_quintic"
    w = bench.workload_by_name("ns_sweep_4096x1024")
    assert w.key == "ns_sweep_4096x1024_cubic" and w.coeffs == "cubic"
    assert bench.workload_by_name("dense_decoder_1p2b").key == "dense_decoder_1p2b"


def test_ns_work_counts_per_slice():
    """Work counts follow each slice's own algorithm: the method's flops do
    not depend on it; Gram space changes only the executed flops and bytes."""
    import workloads as wl
    co = wl.coeff_table("cubic")
    s, l = 2048.0, 5632.0
    sq = [(2048, 2048, False, "gemm128")] * 3
    rect_gs = [(5632, 2048, True, "gemm256")] * 2
    rect_plain = [(5632, 2048, False, "gemm256")] * 2
    a, b, c = bench.ns_work(sq, co, 2), bench.ns_work(rect_gs, co, 2), \
        bench.ns_work(rect_plain, co, 2)
    assert a["method"] == 3 * 5 * 3 * s ** 3 and a["dense"] == 3 * 5 * 4 * s ** 3
    assert a["executed"] == a["method"]
    assert b["method"] == c["method"] == 2 * 5 * 3 * s * s * l
    assert b["executed"] == 2 * (3 * s * s * l + 12 * s ** 3) < c["executed"]
    assert c["bytes"] == 2 * 2 * s * l * 11
    mixed = bench.ns_work(sq + rect_gs, co, 2)
    assert all(mixed[k] == a[k] + b[k] for k in mixed)
    # a quintic row adds s^3 to the method count and 2 s^3 to the dense one
    q = bench.ns_work([(128, 512, True, "resident")], wl.coeff_table("quintic"), 2)
    assert q["method"] == 5 * (3 * 128 * 128 * 512 + 128 ** 3)
    assert q["executed"] == 3 * 128 * 128 * 512 + (12 + 5) * 128 ** 3
    # the fused update replaces the last write by a read and a write of W
    assert bench.ns_work(sq, co, 2, 2)["bytes"] - a["bytes"] == 3 * 2 * s * s
