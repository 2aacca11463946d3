"""Host-side checks of bench.py's reporting (no GPU): the roofline picks the matrix unit or HBM
from the workload's arithmetic intensity, a request for more than one GPU is refused, and the
profile summaries (kernel traces, traffic from FETCH_SIZE / WRITE_SIZE scaled by a plain copy,
counter averages and their derived figures) read rocprofv3's CSV files as documented."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_roofline_long_is_matrix_bound():
    # 16 x 8192 tokens, 16 heads: 1.718e10 visible pairs x 256 FLOP, 1.082 GB algorithmic
    flops = 256 * 16 * 16 * 8192 * 8192
    r = bench.roofline("k", flops, 1082130432, 4.0, None)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["peak"] == bench.PEAK_BF16_TFLOPS
    assert r["achieved"] == pytest.approx(flops / 4e-3 / 1e12, rel=1e-4)
    assert r["frac"] == pytest.approx(r["achieved"] / bench.PEAK_BF16_TFLOPS, abs=1e-4)


def test_roofline_below_the_ridge_is_hbm_bound():
    # 125 FLOP per byte is below 2516.6e12 / 8e12 = 315
    r = bench.roofline("k", 50.7e9, 405_800_000, 0.25, 123)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.PEAK_HBM_GBS
    assert r["achieved"] == pytest.approx(405_800_000 / 0.25e-3 / 1e9, rel=1e-3)
    assert r["traffic"] == 123


def test_ridge_point():
    ridge = bench.PEAK_BF16_TFLOPS * 1e12 / (bench.PEAK_HBM_GBS * 1e9)
    assert bench.roofline("k", ridge * 1000, 1000, 1.0, None)["bound"] == "mfma"
    assert bench.roofline("k", ridge * 999, 1000, 1.0, None)["bound"] == "hbm"


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


NAME_KV = ("void vlf::(anonymous namespace)::back_kv<vlf::(anonymous namespace)::BF16, 4, 2, false>"
           "(unsigned short const*, unsigned short const*, int const*, unsigned int const*)")
NAME_PH = ("void vlf::(anonymous namespace)::attend_pre_ph<vlf::(anonymous namespace)::BF16>"
           "(unsigned short const*, unsigned char const*, float*, int, int, float)")


def _csv(path, header, rows):
    import csv
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def test_short_kernel_name():
    assert bench._short_kernel_name(NAME_KV) == "back_kv<BF16, 4, 2, false>"
    assert bench._short_kernel_name(NAME_PH) == "attend_pre_ph<BF16>"
    assert bench._short_kernel_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_trace_summary_averages_the_last_dispatches(tmp_path, capsys):
    d = tmp_path / "prof"
    d.mkdir()
    _csv(d / "run_kernel_stats.csv",
         ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
          "StdDev"],
         [[NAME_PH, 3, 30000.0, 10000.0, 100.0, 5000.0, 15000.0, 0.0]])
    # three dispatches of 15, 10 and 5 us; the last two are the timed ones
    _csv(d / "run_kernel_trace.csv", ["Dispatch_Id", "Kernel_Name", "Start_Timestamp",
                                      "End_Timestamp"],
         [[1, NAME_PH, 0, 15000], [2, NAME_PH, 20000, 30000], [3, NAME_PH, 40000, 45000]])
    bench.trace_summary([str(d)], timed=2)
    out = capsys.readouterr().out
    assert "attend_pre_ph<BF16> | 3 | 0.030 | 10.00 | 5.00 | 15.00 | 100.00" in out
    assert "attend_pre_ph<BF16> | timed_average_us 7.50 | over 2" in out
    assert f"kernel_source_sha256_16: {bench.kernel_hash()}" in out


def test_traffic_is_scaled_by_the_plain_copy(tmp_path, capsys):
    # the copy of COPY_BYTES reads as half its size in FETCH_SIZE and as its size in WRITE_SIZE
    # (KiB): scale factors 2 and 1
    fetch, write = tmp_path / "f", tmp_path / "w"
    fetch.mkdir()
    write.mkdir()
    head = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    kib = bench.COPY_BYTES / 1024
    _csv(fetch / "run_counter_collection.csv", head,
         [[1, NAME_PH, "FETCH_SIZE", 1000.0], [2, NAME_PH, "FETCH_SIZE", 3000.0],
          [3, "__amd_rocclr_copyBuffer", "FETCH_SIZE", kib / 2]])
    _csv(write / "run_counter_collection.csv", head,
         [[1, NAME_PH, "WRITE_SIZE", 500.0], [3, "__amd_rocclr_copyBuffer", "WRITE_SIZE", kib]])
    bench.summarize([str(fetch), str(write)], "long", "attend_pre_ph")
    lines = dict(line.split(": ", 1) for line in capsys.readouterr().out.splitlines())
    assert float(lines["FETCH_SIZE_scale_factor"]) == pytest.approx(2.0)
    assert float(lines["hbm_fetch_bytes_per_launch"]) == pytest.approx(2000 * 1024 * 2)
    assert float(lines["hbm_write_bytes_per_launch"]) == pytest.approx(500 * 1024)
    assert float(lines["hbm_bytes_per_launch"]) == pytest.approx(2000 * 2048 + 500 * 1024)


def test_counters_derive_busy_fractions(tmp_path, capsys):
    d = tmp_path / "c"
    d.mkdir()
    xcd_cycles = 1000.0
    rows = [[1, NAME_PH, "GRBM_GUI_ACTIVE", 8 * xcd_cycles],
            [1, NAME_PH, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * xcd_cycles * 1024],
            [1, NAME_PH, "SQ_INSTS_MFMA", 0.5 * xcd_cycles * 1024 / 32],
            [1, NAME_PH, "SQ_INSTS_VALU", 3 * 0.5 * xcd_cycles * 1024 / 32],
            [1, NAME_PH, "SQ_WAVE_CYCLES", 2 * 256 * xcd_cycles],
            [1, NAME_PH, "SQ_WAIT_ANY", 0.25 * 2 * 256 * xcd_cycles]]
    _csv(d / "run_counter_collection.csv",
         ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    bench.counters([str(d)], "long", "attend_pre_ph")
    out = dict(line.split(": ", 1) for line in capsys.readouterr().out.splitlines()
               if ": " in line)
    assert float(out["mfma_busy_pct_of_simd_cycles"]) == pytest.approx(50.0)
    assert float(out["mfma_busy_cycles_per_mfma"]) == pytest.approx(32.0)
    assert float(out["non_mfma_valu_insts_per_mfma"]) == pytest.approx(2.0)
    # SQ_WAVE_CYCLES counts quad-cycles: 2 per CU-cycle is 8 waves resident
    assert float(out["waves_resident_per_cu"]) == pytest.approx(8.0)
    assert float(out["SQ_WAIT_ANY_pct_of_wave_cycles"]) == pytest.approx(25.0)


def test_traffic_is_read_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    path = tmp_path / "k_long_traffic.txt"
    monkeypatch.setattr(bench, "traffic_file", lambda kernel, workload: str(path))
    assert bench.read_traffic("k", "long") is None
    path.write_text(f"# header\nkernel_source_sha256_16: {bench.kernel_hash()}\n"
                    "hbm_bytes_per_launch: 1234\n")
    assert bench.read_traffic("k", "long") == 1234.0
    path.write_text("kernel_source_sha256_16: 0000000000000000\nhbm_bytes_per_launch: 1234\n")
    assert bench.read_traffic("k", "long") is None
