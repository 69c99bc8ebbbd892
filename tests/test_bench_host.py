"""Host-side checks of bench.py (no GPU): the roofline it reports and the
one-GPU restriction."""
import os
import subprocess
import sys

import pytest

import bench
from flashattention_forward_tile_amd.workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_headline_roofline_is_the_matrix_core_roof():
    w = WORKLOADS["headline"]
    assert w.flops == 4 * 4 * 16 * 4096 * 4096 * 128
    r = bench.roofline_of(w, 0.5, None)  # 0.5 ms per launch
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2516.6
    assert r["achieved"] == pytest.approx(w.flops / 0.5e-3 / 1e12, rel=1e-6)
    assert r["frac"] == pytest.approx(r["achieved"] / 2516.6, abs=1e-4)


@pytest.mark.parametrize("name", ["sweep_n512", "gqa_chunk", "tiny"])
def test_short_workloads_sit_under_the_hbm_roof(name):
    """Arithmetic intensity below 2516.6 TFLOP/s / 8 TB/s = 315 FLOP/B."""
    w = WORKLOADS[name]
    assert w.flops / w.algo_bytes < 315.0
    r = bench.roofline_of(w, 0.1, 12345)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(w.algo_bytes / 0.1e-3 / 1e9, abs=0.05)
    assert r["traffic"] == 12345


def test_every_other_workload_is_matrix_bound():
    for name, w in WORKLOADS.items():
        if name in ("sweep_n512", "gqa_chunk", "tiny"):
            continue
        assert bench.roofline_of(w, 1.0, None)["bound"] == "mfma", name


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
