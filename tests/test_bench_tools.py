"""CPU tests of bench.py's measurement tooling, on synthetic rocprofv3 csv files: the source hash
that gates the reported traffic, the traffic summary (copy calibration, per-kernel means, the
hash stamp) with its reader, the labelled per-kernel counter summary and the kernel-trace
summary's cutting of a trace into calls."""
import csv
import os

import bench


def _write_counters(d, counter, rows):
    """rocprofv3-style counter csv; each value split over two rows, as counters reported per
    dimension are, so that the readers' per-dispatch sums are exercised."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for disp, name, val in rows:
            w.writerow([disp, name, counter, val / 2])
            w.writerow([disp, name, counter, val / 2])


def test_source_hash_ignores_comments_and_layout(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ["k.hip"])
    src.write_text("int f(int a) { return a + 1; }  // one\n/* block */\n")
    h0 = bench.kernel_source_hash()
    src.write_text("int f(int a) {\n  return a + 1;  // another comment\n}\n/* and\n another */\n")
    assert bench.kernel_source_hash() == h0
    src.write_text("int f(int a) { return a + 2; }\n")
    assert bench.kernel_source_hash() != h0


def test_traffic_summary_and_reader(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.txt"))
    copy_kib = bench.COPY_BYTES / 1024
    gate_up = "void beam::gateup_stream_lds_kernel<3, 128, 8>(int)"
    grouped = "void beam::grouped_gemm_kernel<true, false, false>(int)"
    calib = "void at::native::neg_kernel(int)"
    # FETCH_SIZE reads half the calibration copy's bytes (scale 2), WRITE_SIZE all of them (scale 1)
    _write_counters(tmp_path / "fetch" / "sub", "FETCH_SIZE",
                    [(1, calib, copy_kib / 2), (2, gate_up, 1000.0), (3, gate_up, 3000.0), (4, grouped, 500.0)])
    _write_counters(tmp_path / "write", "WRITE_SIZE",
                    [(1, calib, copy_kib), (2, gate_up, 10.0), (3, gate_up, 30.0), (4, grouped, 7.0)])
    bench.summarize_pmc(str(tmp_path / "fetch"), str(tmp_path / "write"))
    # per launch: (mean fetch KiB * 2 + mean write KiB * 1) * 1024 bytes
    assert bench.measured_traffic("decode") == (2000 * 2 + 20) * 1024
    assert bench.measured_traffic("prefill") == (500 * 2 + 7) * 1024
    assert bench.measured_traffic("decode_fp8") is None  # no dispatch of that kernel in the runs
    # a figure taken on other kernel sources is not reported
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.measured_traffic("decode") is None


def test_counter_summary_keeps_passes_apart(tmp_path):
    grouped = "void beam::grouped_gemm_kernel<true, false, false>(int)"
    for label, busy in (("prefill", 0.5), ("skewed", 0.25)):
        d = tmp_path / label
        os.makedirs(d)
        with open(d / "run_counter_collection.csv", "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            # MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs)
            w.writerow([1, grouped, "GRBM_GUI_ACTIVE", 8 * 200])
            w.writerow([1, grouped, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 200 * busy / 2])
            w.writerow([1, grouped, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 200 * busy / 2])
            w.writerow([1, grouped, "SQ_WAIT_ANY", 30])
            w.writerow([1, grouped, "SQ_WAVE_CYCLES", 100])
    out = tmp_path / "summary.md"
    bench.summarize_counters(str(out), f"prefill={tmp_path / 'prefill'}", f"skewed={tmp_path / 'skewed'}")
    text = out.read_text()
    prefill = text[text.index("## prefill: `beam::grouped_gemm_kernel<true, false, false>` (1 dispatches)"):
                   text.index("## skewed:")]
    skewed = text[text.index("## skewed: `beam::grouped_gemm_kernel<true, false, false>` (1 dispatches)"):]
    assert "| MFMA busy (derived) | 0.500 |" in prefill and "| MFMA busy (derived) | 0.250 |" in skewed
    assert "| wave wait (derived) | 0.300 |" in prefill
    assert "--workloads prefill " in text and "--workloads skewed " in text


def test_trace_summary_cuts_and_classifies_calls(tmp_path):
    """Five calls in a row (decode, prefill, FP8 decode, a residual-sublayer decode, prefill with
    packed down weights): each is cut at
    its router (or its prenorm) and filed under its workload; other kernels are ignored."""
    calls = [
        ["router_logits_kernel<64>", "select_kernel", "dispatch_small_kernel", "gateup_stream_lds_kernel<3, 128, 8>",
         "down_stream_lds_kernel<3, 128, 8, 1, false>", "combine_kernel"],
        ["router_logits_kernel<128>", "select_kernel", "dispatch_hist_kernel", "dispatch_scan_kernel",
         "dispatch_scatter_kernel", "grouped_gemm_kernel<true, false, false>", "grouped_gemm_kernel<false, false, false>",
         "combine_kernel"],
        ["router_logits_kernel<64>", "select_kernel", "dispatch_small_kernel", "gateup_stream_fp8_kernel<3, 8>",
         "down_stream_fp8_kernel<3, 8, 1>", "combine_kernel"],
        ["prenorm_kernel", "router_logits_kernel<64>", "select_kernel", "dispatch_small_kernel",
         "gateup_stream_lds_kernel<3, 128, 8>", "down_stream_lds_kernel<3, 128, 8, 1, false>", "combine_residual_kernel"],
        ["router_logits_kernel<128>", "select_kernel", "dispatch_hist_kernel", "dispatch_scan_kernel",
         "dispatch_scatter_kernel", "grouped_gemm_kernel<true, false, false>", "grouped_gemm_kernel<false, false, true>",
         "combine_kernel"],
    ]
    os.makedirs(tmp_path / "trace" / "host")
    t = 1000
    with open(tmp_path / "trace" / "host" / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for ci, c in enumerate(calls):
            for ki, k in enumerate(c):
                dur = 1000 * (ci + 1) + 100 * ki  # ns
                w.writerow([f"void beam::{k}(int)", t, t + dur])
                t += dur + 50
            w.writerow(["void at::native::fill_kernel(int)", t, t + 5])  # not the library's
            t += 100
    out = tmp_path / "kernels.md"
    bench.summarize_trace(str(tmp_path / "trace"), str(out))
    text = out.read_text()
    sections = {s.split("\n", 1)[0]: s for s in text.split("\n## ")[1:]}
    assert set(sections) == {"decode", "prefill", "decode_fp8", "decode, residual sublayer", "prefill_packed"}
    assert "`beam::grouped_gemm_kernel<false, false, true>` | 1 | 5.6 |" in sections["prefill_packed"]
    # each call's kernels are filed under its own workload, with its own durations (1 us per call
    # index, plus 0.1 us per position in the call)
    assert "`beam::grouped_gemm_kernel<true, false, false>` | 1 | 2.5 |" in sections["prefill"]
    assert "`beam::gateup_stream_fp8_kernel<3, 8>` | 1 | 3.3 |" in sections["decode_fp8"]
    assert "`beam::prenorm_kernel` | 1 | 4.0 |" in sections["decode, residual sublayer"]
    assert "`beam::router_logits_kernel<64>` | 1 | 4.1 |" in sections["decode, residual sublayer"]
    assert "`beam::combine_kernel` | 1 | 1.5 |" in sections["decode"]
    assert "fill_kernel" not in text


def test_bench_refuses_more_than_one_gpu():
    """The block runs on one GPU: --gpus N with N > 1 (or a multi-rank launch) exits with status 2
    and says why, before anything touches a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for args, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *args], capture_output=True, text=True,
                           env={**os.environ, **env}, timeout=120)
        assert r.returncode == 2, r.stderr
        assert "one GPU" in r.stderr
        assert r.stdout == ""
