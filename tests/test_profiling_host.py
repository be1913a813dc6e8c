"""Host logic of the counter summaries (adamw_optimizer_step_amd.profiling):
copy calibration, kernel-name matching, MfmaUtil averaging and the written
summary, on synthetic rocprofv3 counter files."""

import contextlib
import csv
import io

import pytest

from adamw_optimizer_step_amd import profiling

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
GEMM = "void mo::(anonymous namespace)::k_ns_gemm<unsigned short, 256, 256, 2, 4, 2, true>(x)"
MOM = "void mo::(anonymous namespace)::k_momentum<true>(mo::MomSeg const*, int)"
COPY = "mo::(anonymous namespace)::k_diag_copy(unsigned int const*, unsigned int*, long)"
OTHER = "void mo::(anonymous namespace)::k_ns_gemm_helper(int)"


def _csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d, name, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": v})


@pytest.fixture
def counters(tmp_path):
    mib = 1 << 20
    # the copy of 1 MiB is counted as 512 KiB fetched and 1024 KiB written;
    # two GEMM launches listed out of dispatch order; a name that only starts
    # like the kernel's must not match
    fetch, write, mfma = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "m.csv"
    _csv(fetch, "FETCH_SIZE", [(7, GEMM, 300.0), (1, COPY, 512.0), (3, GEMM, 100.0),
                               (5, OTHER, 9999.0), (2, MOM, 64.0)])
    _csv(write, "WRITE_SIZE", [(1, COPY, 1024.0), (3, GEMM, 40.0), (7, GEMM, 60.0),
                               (5, OTHER, 9999.0), (2, MOM, 128.0)])
    _csv(mfma, "MfmaUtil", [(3, GEMM, 50.0), (7, GEMM, 54.0), (5, OTHER, 99.0)])
    return mib, str(fetch), str(write), str(mfma)


def test_summary_scales_by_the_copy(counters):
    mib, f, w, m = counters
    s = profiling.counters_summary("wl", "quintic", "bf16", mib, f, w, m)
    assert s["scale_fetch"] == pytest.approx(2.0)
    assert s["scale_write"] == pytest.approx(1.0)
    g = s["kernels"]["k_ns_gemm"]
    assert g["launches"] == 2
    # mean counted KiB x 1024 x scale
    assert g["fetch_bytes_per_launch"] == pytest.approx(2.0 * 200.0 * 1024)
    assert g["write_bytes_per_launch"] == pytest.approx(50.0 * 1024)
    assert g["mfma_util_pct"] == pytest.approx(52.0)
    assert g["source_digest"] == profiling.source_digest("k_ns_gemm")
    k = s["kernels"]["k_momentum"]
    assert k["fetch_bytes_per_launch"] == pytest.approx(2.0 * 64.0 * 1024)
    assert "mfma_util_pct" not in k
    assert set(s["kernels"]) == {"k_ns_gemm", "k_momentum"}


def test_per_dispatch_order(counters):
    _, f, _, _ = counters
    t = profiling._per_dispatch(f, "FETCH_SIZE")
    assert t[GEMM] == [100.0, 300.0]
    assert profiling._match(t, "k_ns_gemm") == [100.0, 300.0]
    assert profiling._match(t, "k_diag_copy") == [512.0]


def test_missing_calibration_is_an_error(tmp_path, counters):
    mib, f, w, _ = counters
    bad = tmp_path / "nocopy.csv"
    _csv(bad, "FETCH_SIZE", [(3, GEMM, 100.0)])
    with pytest.raises(SystemExit):
        profiling.counters_summary("wl", "cubic", "bf16", mib, str(bad), w)


def test_written_summary_reads_back(counters, tmp_path):
    mib, f, w, m = counters
    out = io.StringIO()
    with contextlib.redirect_stdout(out):
        rc = profiling.main(["counters", "--workload", "wl", "--copy-bytes", str(mib),
                             "--fetch", f, "--write", w, "--mfma", m, "--command", "a b;;c d"])
    assert rc == 0
    path = tmp_path / profiling.summary_name("wl", "cubic", "bf16")
    path.write_text(out.getvalue())
    s = profiling.read_summary(str(path))
    assert s["workload"] == "wl" and s["coeffs"] == "cubic" and s["precision"] == "bf16"
    assert float(s["kernels"]["k_ns_gemm"]["fetch_bytes_per_launch"]) == pytest.approx(409600.0)
    # the command lines are indented and not parsed as keys
    assert "    a b" in out.getvalue() and "    c d" in out.getvalue()
    g = profiling.kernel_figures(str(path), "k_ns_gemm", "wl", "cubic", "bf16")
    assert g["mfma_util_pct"] == pytest.approx(52.0) and g["launches"] == 2
    # another configuration, or a kernel the summary lacks: no figures
    assert profiling.kernel_figures(str(path), "k_ns_gemm", "wl", "quintic", "bf16") is None
    assert profiling.kernel_figures(str(path), "k_rows", "wl", "cubic", "bf16") is None
    assert profiling.read_summary(str(tmp_path / "absent.md")) is None


def test_stale_digest_gives_no_figures(counters, tmp_path):
    mib, f, w, m = counters
    out = io.StringIO()
    profiling.write_summary(profiling.counters_summary("wl", "cubic", "bf16", mib, f, w, m),
                            [], out)
    text = out.getvalue().replace(profiling.source_digest("k_ns_gemm"), "0123456789abcdef")
    path = tmp_path / "s.md"
    path.write_text(text)
    assert profiling.kernel_figures(str(path), "k_ns_gemm", "wl", "cubic", "bf16") is None
    assert profiling.kernel_figures(str(path), "k_momentum", "wl", "cubic", "bf16") is not None
