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


def test_ns_work_applies_gram_space_per_slice():
    """Gram space covers rectangular GEMM slices and slice-resident ones with
    a short side of 64 or more; the others count as the plain iteration."""
    import workloads as wl
    co = wl.coeff_table("cubic")
    sq, rect = [(2048, 2048)] * 3, [(5632, 2048)] * 2
    plain_sq = bench.ns_work(sq, co, 2)
    assert bench.ns_work(sq, co, 2, gram_space=True) == plain_sq
    gs_rect = bench.ns_work(rect, co, 2, gram_space=True)
    assert gs_rect != bench.ns_work(rect, co, 2)
    mixed = bench.ns_work(sq + rect, co, 2, gram_space=True)
    assert mixed == tuple(a + b for a, b in zip(plain_sq, gs_rect))
    # square slices execute the same flops in either form (N = 5, cubic)
    s = 2048.0
    assert plain_sq[1] == 3 * 15 * s ** 3
    small = [(32, 512), (128, 512)]
    got = bench.ns_work(small, co, 2, gram_space=True, sxs_on_chip=True)
    want = [bench.ns_work([small[0]], co, 2), bench.ns_work([small[1]], co, 2, gram_space=True,
                                                             sxs_on_chip=True)]
    assert got == tuple(a + b for a, b in zip(*want))
