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
