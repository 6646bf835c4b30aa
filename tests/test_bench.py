"""The benchmark's host-side contract (no GPU): refusal of several GPUs, the
PMC traffic summary, and the rule that a stored traffic figure is used only for
the kernel source it was measured on."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_kernel_names_follow_the_tile():
    base = dict(lanes_per_row=32, rows_per_batch=4, waves_per_wg=5, k_slice=512, rows_per_wg=40, mfma=0, kind=2, depth=2)
    assert bench.kernel_name(base, 1) == "qgemv_dma_kernel<0, 1, 8, 2, false>"
    assert bench.kernel_name(dict(base, kind=3, depth=3), 4) == "qgemv_dma_kernel<0, 4, 8, 3, true>"
    assert bench.kernel_name(dict(base, kind=1, depth=0), 2) == "qgemv_stream_kernel<0, 2, 8>"
    assert bench.kernel_name(dict(base, kind=1, depth=0, rows_per_batch=8, mfma=1), 3) == "qgemv_mfma_q8_kernel<3>"
    assert bench.kernel_name(dict(base, kind=1, depth=0, rows_per_batch=8, mfma=2), 4) == "qgemv_mfma_persist_kernel<4>"
    assert bench.kernel_name(dict(base, kind=4, depth=3), 2) == "qgemv_units_kernel<0, 2, 3>"
    assert bench.kernel_name(dict(base, kind=0, depth=0, rows_per_wg=8), 1) == "qgemv_dense_kernel<0, 1, 4, true>"
    assert bench.kernel_name(dict(base, kind=7, waves_per_wg=10, depth=2), 4) == "qgemv_half_kernel<0, 4, 2>"
    assert bench.kernel_name(dict(base, kind=8, waves_per_wg=10, depth=1), 3) == "qgemv_mx_kernel<0, 3, 1, 1>"
    assert bench.kernel_name(dict(base, kind=8, waves_per_wg=10, depth=2), 1) == "qgemv_mx_kernel<0, 1, 2, 1>"
    assert bench.kernel_name(dict(base, kind=11, waves_per_wg=12, depth=1), 2) == "qgemv_mx_kernel<0, 2, 1, 2>"
    assert bench.kernel_name(dict(base, kind=9, waves_per_wg=10, depth=1), 4) == "qgemv_mxp_kernel<0, 4>"


def _write_pmc(dirpath, counter, rows):
    os.makedirs(dirpath, exist_ok=True)
    with open(os.path.join(dirpath, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for disp, name, value in rows:
            w.writerow(dict(Dispatch_Id=disp, Kernel_Name=name, Counter_Name=counter, Counter_Value=value))


def test_pmc_summary_scales_by_the_copy_calibration(tmp_path, capsys):
    nbytes = 27852800
    copy = "at::native::vectorized_elementwise_kernel<4, MulFunctor<float>>"
    k = "void qg::(anonymous namespace)::qgemv_dma_kernel<0, 1, 8, 2, false>(qg::DenseArgs)"
    # FETCH_SIZE reads half the true bytes for the copy; two dispatches each, split over two XCD rows
    _write_pmc(tmp_path / "f", "FETCH_SIZE", [(1, copy, nbytes / 2048 / 2), (1, copy, nbytes / 2048 / 2),
                                             (2, k, 7000.0), (2, k, 7000.0), (3, k, 6000.0), (3, k, 8000.0)])
    _write_pmc(tmp_path / "w", "WRITE_SIZE", [(1, copy, nbytes / 1024), (2, k, 40.0), (3, k, 40.0)])
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), nbytes)
    out = capsys.readouterr().out
    row = [line for line in out.splitlines() if line.startswith("| qgemv_dma_kernel")]
    assert len(row) == 1
    cells = [c.strip() for c in row[0].strip("|").split("|")]
    assert float(cells[1]) == 14000.0                   # per-dispatch sum, median over dispatches
    assert int(cells[3]) == 2 * 14000 * 1024            # scaled by 2: the copy's FETCH_SIZE reads half
    assert int(cells[4]) == 2 * 14000 * 1024 + 40 * 1024


def test_stored_traffic_needs_the_same_kernel_source(tmp_path, monkeypatch):
    f = tmp_path / "t.txt"
    f.write_text("kernel_source_sha256: %s\n\n| kernel | a | b | c | d | e |\n|---|---|---|---|---|---|\n"
                 "| qgemv_x<1> | 1 | 2 | 3 | 12345 | 1.0 |\n" % bench.source_digest())
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("qgemv_x<1>") == 12345
    assert bench.measured_traffic("qgemv_y<1>") is None
    f.write_text(f.read_text().replace(bench.source_digest(), "0" * 16))
    assert bench.measured_traffic("qgemv_x<1>") is None


def test_trace_and_counter_summaries(tmp_path, capsys):
    d = tmp_path / "t"
    d.mkdir()
    (d / "run_kernel_stats.csv").write_text(
        "Name,Calls,TotalDurationNs,AverageNs,Percentage,MinNs,MaxNs,StdDev\n"
        '"void qg::(anonymous namespace)::qgemv_dma_kernel<0, 1, 8, 2, false>(unsigned char const*)",10,80000,8000.0,'
        "60.0,7000,9000,10\n"
        '"at::native::elementwise_kernel",5,100,20.0,1.0,10,30,1\n')
    bench.summarize_trace(str(d))
    out = capsys.readouterr().out
    assert "| qgemv_dma_kernel<0, 1, 8, 2, false> | 10 | 8.000 | 7.000 | 9.000 | 60.00% |" in out
    assert "elementwise" not in out
    _write_pmc(tmp_path / "c", "SQ_WAVES", [(1, "void qg::(anonymous namespace)::qgemv_x<1>(a)", 5.0),
                                            (1, "void qg::(anonymous namespace)::qgemv_x<1>(a)", 7.0),
                                            (2, "void qg::(anonymous namespace)::qgemv_x<1>(a)", 100.0)])
    bench.summarize_counters(str(tmp_path / "c"))
    out = capsys.readouterr().out
    assert "| qgemv_x<1> | 100 |" in out  # per-dispatch sums (12, 100): the median of two is the upper


def test_clock_fields_keep_clocks_and_power():
    doc = [{"gpu": 0, "power": {"socket_power": {"value": 512, "unit": "W"}},
            "clock": {"gfx_0": {"clk": {"value": 2100, "unit": "MHz"}, "min_clk": {"value": 500}},
                      "mem_0": {"clk": {"value": 1900, "unit": "MHz"}}, "vclk_0": {"clk": {"value": 29}}}}]
    got = bench.clock_fields(doc)
    assert got == {"[0].power.socket_power.value": 512, "[0].clock.gfx_0.clk.value": 2100,
                   "[0].clock.mem_0.clk.value": 1900}


def test_clock_sample_never_raises():
    assert isinstance(bench.gpu_clocks(), dict)  # without a GPU: the reason, not an exception


def test_no_clock_sampling_under_the_profiler(monkeypatch):
    """amd-smi is a script started through env: under rocprofv3 its process would
    inherit the tool library, so the bench takes no sample there."""
    monkeypatch.setenv("LD_PRELOAD", "/opt/rocm/lib/rocprofiler-sdk/librocprofiler-sdk-tool.so")
    assert bench.gpu_clocks() == {"skipped": "under rocprofv3"}
    assert bench.clocks_under_load(None, lambda: None, 0.0) == {"skipped": "under rocprofv3"}


def test_trace_summary_leaves_out_the_first_dispatches(tmp_path, capsys):
    # dispatches listed out of order: the summary sorts them by start time, drops the
    # first N of this library's kernels (other kernels neither count nor show) and
    # aggregates the rest per kernel
    d = tmp_path / "t"
    d.mkdir()
    name_a = '"void qg::(anonymous namespace)::qgemv_mxp_kernel<0, 1>(qg::DenseArgs)"'
    name_b = '"void qg::(anonymous namespace)::qgemv_mxp_kernel<0, 2>(qg::DenseArgs)"'
    rows = [(name_a, 3000, 3004), (name_a, 1000, 1009), ('"at::native::copy_kernel"', 500, 900),
            (name_a, 2000, 2005), (name_b, 4000, 4006), (name_b, 5000, 5008)]
    (d / "run_kernel_trace.csv").write_text(
        "Kernel_Name,Start_Timestamp,End_Timestamp\n" + "".join(f"{n},{s},{e}\n" for n, s, e in rows))
    bench.summarize_trace(str(d), skip_first=1)
    out = capsys.readouterr().out
    # qgemv_mxp_kernel<0, 1> keeps the dispatches at 2000 (5 ns) and 3000 (4 ns)
    assert "| qgemv_mxp_kernel<0, 1> | 2 | 0.005 | 0.004 | 0.005 | 39.13% |" in out
    assert "| qgemv_mxp_kernel<0, 2> | 2 | 0.007 | 0.006 | 0.008 | 60.87% |" in out
    assert "copy_kernel" not in out
    assert "share of this library's kernel time" in out
