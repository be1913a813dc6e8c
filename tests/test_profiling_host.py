"""Host logic of the counter summaries (adamw_optimizer_step_amd.profiling):
copy calibration, kernel-name matching and the written summary, on synthetic
rocprofv3 counter files."""

import csv
import io
import contextlib

import pytest

from adamw_optimizer_step_amd import profiling

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
GEMM = "void mo::(anonymous namespace)::k_ns_gemm<unsigned short, 256, 256, 2, 4, 2, true>(x)"
COPY = "mo::(anonymous namespace)::k_diag_copy(unsigned int const*, unsigned int*, long)"
OTHER = "void mo::(anonymous namespace)::k_ns_gemm_helper(int)"


def _csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d, name, kib in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": kib})


@pytest.fixture
def counters(tmp_path):
    mib = 1 << 20
    # the copy of 1 MiB is counted as 512 KiB fetched and 1024 KiB written;
    # two GEMM launches, listed out of dispatch order; a name that only
    # starts like the kernel's must not match
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    _csv(fetch, "FETCH_SIZE", [(7, GEMM, 300.0), (1, COPY, 512.0), (3, GEMM, 100.0),
                               (5, OTHER, 9999.0)])
    _csv(write, "WRITE_SIZE", [(1, COPY, 1024.0), (3, GEMM, 40.0), (7, GEMM, 60.0),
                               (5, OTHER, 9999.0)])
    return mib, str(fetch), str(write)


def test_traffic_summary_scales_by_the_copy(counters):
    mib, f, w = counters
    s = profiling.traffic_summary("k_ns_gemm", "wl", mib, f, w, "quintic", "bf16")
    assert s["launches"] == 2
    assert s["scale_fetch"] == pytest.approx(2.0)
    assert s["scale_write"] == pytest.approx(1.0)
    # mean counted KiB x 1024 x scale
    assert s["fetch_bytes_per_launch"] == pytest.approx(2.0 * 200.0 * 1024)
    assert s["write_bytes_per_launch"] == pytest.approx(50.0 * 1024)
    assert s["coeffs"] == "quintic" and s["precision"] == "bf16"
    assert s["source_digest"] == profiling.source_digest("k_ns_gemm")


def test_per_dispatch_order(counters):
    _, f, _ = counters
    t = profiling._per_dispatch(f, "FETCH_SIZE")
    assert t[GEMM] == [100.0 * 1024, 300.0 * 1024]
    assert profiling._match(t, "k_ns_gemm") == [100.0 * 1024, 300.0 * 1024]
    assert profiling._match(t, "k_diag_copy") == [512.0 * 1024]


def test_missing_kernel_is_an_error(counters):
    mib, f, w = counters
    with pytest.raises(SystemExit):
        profiling.traffic_summary("k_ns_small", "wl", mib, f, w)


def test_written_summary_reads_back(counters, tmp_path):
    mib, f, w = counters
    out = io.StringIO()
    with contextlib.redirect_stdout(out):
        rc = profiling.main(["traffic", "--kernel", "k_ns_gemm", "--workload", "wl",
                             "--coeffs", "cubic", "--copy-bytes", str(mib), "--fetch", f,
                             "--write", w, "--command", "a b;;c d"])
    assert rc == 0
    path = tmp_path / "s.md"
    path.write_text(out.getvalue())
    s = profiling.read_summary(str(path))
    assert s["kernel"] == "k_ns_gemm" and s["workload"] == "wl"
    assert s["coeffs"] == "cubic" and s["precision"] == "bf16"
    assert float(s["fetch_bytes_per_launch"]) == pytest.approx(409600.0)
    # the command lines are indented and not parsed as keys
    assert "a b" in out.getvalue() and "    c d" in out.getvalue()
    assert profiling.read_summary(str(tmp_path / "absent.md")) is None
