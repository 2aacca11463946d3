"""Host-side checks of bench.py's reporting (no GPU): the roofline picks the matrix unit or HBM
from the workload's arithmetic intensity, and a request for more than one GPU is refused."""
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
