"""Host logic of bench.py, no GPU: the counter summaries (HBM traffic from
FETCH_SIZE / WRITE_SIZE scaled by a copy calibration; clock and MFMA activity
of the prefill GEMMs), the rule that a committed traffic figure is used only
for the kernel source it was taken on, and the one-GPU limit of the bench."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import synth  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _row(disp, kernel, counter, value, t0=0, t1=1000):
    return {"Dispatch_Id": disp, "Kernel_Name": kernel, "Counter_Name": counter,
            "Counter_Value": value, "Start_Timestamp": t0, "End_Timestamp": t1}


def test_traffic_summary_scales_by_the_copy(tmp_path):
    gib_kib = 1 << 20
    kern = "up_decode_kernel<1>"
    full = f"moe::(anonymous namespace)::{kern}(unsigned char const*, int)"
    copy = "__amd_rocclr_copyBuffer"
    # the copy of 1 GiB reads as half a GiB of FETCH_SIZE and a whole GiB of WRITE_SIZE
    fetch = [_row(i, copy, "FETCH_SIZE", gib_kib / 2) for i in range(3)]
    fetch += [_row(10 + i, full, "FETCH_SIZE", 1000.0 + 10 * i) for i in range(3)]   # mean 1010 KiB
    write = [_row(i, copy, "WRITE_SIZE", gib_kib) for i in range(3)]
    write += [_row(10 + i, full, "WRITE_SIZE", 50.0) for i in range(3)]
    _write_counters(tmp_path / "f", fetch)
    _write_counters(tmp_path / "w", write)
    text = bench.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), kern, "wl", "c1", 20)
    got = float([ln for ln in text.splitlines() if ln.startswith("- traffic_bytes_per_launch: ")][0].split(": ")[1])
    assert got == pytest.approx((1010.0 * 2 + 50.0) * 1024)
    assert "scale factors 2.0000 / 1.0000" in text


def test_traffic_summary_names_missing_kernels(tmp_path):
    _write_counters(tmp_path / "f", [_row(0, "other_kernel(int)", "FETCH_SIZE", 1.0)])
    _write_counters(tmp_path / "w", [_row(0, "other_kernel(int)", "WRITE_SIZE", 1.0)])
    with pytest.raises(SystemExit, match="missing kernels"):
        bench.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), "up_decode_kernel<1>", "wl")


def test_mfma_summary_clock_busy_and_rate(tmp_path):
    sh = synth.CONFIGS["c3"]
    rows = []
    for kern, flops in bench.MFMA_KERNELS.items():
        full = f"void moe::(anonymous namespace)::{kern}(moe::(anonymous namespace)::KArgs)"
        ns = 1_000_000                                   # 1 ms per launch
        cyc = 2.0e9 * 1e-3                               # 2.0 GHz on each XCD
        for d in range(2):
            disp = f"{kern}-{d}"
            rows.append(_row(disp, full, "GRBM_GUI_ACTIVE", cyc * bench.N_XCD, 0, ns))
            rows.append(_row(disp, full, "SQ_BUSY_CYCLES", 1.0, 0, ns))
            rows.append(_row(disp, full, "SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * cyc * bench.N_SIMD, 0, ns))
    _write_counters(tmp_path / "m", rows)
    text = bench.mfma_summary(str(tmp_path / "m"), "wl", "c3", 6)
    lines = {ln.split("|")[1].strip(): [c.strip() for c in ln.split("|")[2:-1]]
             for ln in text.splitlines() if ln.startswith("| prefill_gemm")}
    for kern, flops in bench.MFMA_KERNELS.items():
        disp, dur, ghz, busy, pf, of_peak, of_clk = lines[kern]
        assert disp == "2" and dur == "1000.0" and ghz == "2.00" and busy == "25.0 %"
        rate = flops(sh) / 1e-3 / 1e15
        assert float(pf) == pytest.approx(rate, abs=0.006)
        assert float(of_clk.rstrip(" %")) == pytest.approx(100 * rate / (5.0 * 2.0 / 2.4), abs=0.06)
    # the gate/up GEMM does twice the down GEMM's multiply-adds (W1 and W3)
    assert bench.MFMA_KERNELS["prefill_gemm_kernel<true>"](sh) == 2 * bench.MFMA_KERNELS["prefill_gemm_kernel<false>"](sh)
    assert bench.MFMA_KERNELS["prefill_gemm_kernel<false>"](sh) == 2.0 * sh.H * sh.I * sh.T * sh.k


def test_traffic_figure_needs_the_current_source(tmp_path, monkeypatch):
    kern = "up_decode_kernel<1>"
    src = tmp_path / "kernel.hip"
    src.write_text("// version 1\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setitem(bench.KERNEL_SOURCES, kern, "kernel.hip")
    summary = tmp_path / "profiles" / "k_traffic.md"
    summary.write_text(f"# HBM traffic: {kern}, wl\n\n- source_sha256: {bench.source_sha256(kern)}\n"
                       "- traffic_bytes_per_launch: 12345\n")
    assert bench.load_traffic(kern, "wl") == 12345.0
    assert bench.load_traffic(kern, "another workload") is None
    src.write_text("// version 2\n")                     # the kernel changed since the counters were taken
    assert bench.load_traffic(kern, "wl") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
