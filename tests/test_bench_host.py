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


HBM_BOUND = ("sweep_n512", "gqa_chunk", "tiny", "decode", "decode_long", "decode_int8",
             "decode_fp8")


@pytest.mark.parametrize("name", HBM_BOUND)
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
        if name in HBM_BOUND:
            continue
        assert bench.roofline_of(w, 1.0, None)["bound"] == "mfma", name


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_bench_parity_against_the_oracle_on_the_cpu():
    """The parity object of the bench line, fed outputs made on the CPU: the
    oracle's own result rounded to bf16 passes; the same with one element
    moved by 0.05 fails (and the error is the one planted)."""
    import numpy as np
    import torch

    import oracle
    from flashattention_forward_tile_amd.workloads import bits, workload_inputs

    w = WORKLOADS["tiny"]
    q, k, v = workload_inputs(w, seed=0)
    o_ref, lse_ref = oracle.attention(bits(q), bits(k), bits(v), w.dtype, w.scale)
    o = torch.from_numpy(o_ref).to(torch.bfloat16)
    lse = torch.from_numpy(lse_ref).to(torch.float32)
    base, par = bench.cpu_baseline(w, q, k, v, o, lse)
    assert base["kind"] == "oracle" and base["cores"] >= 1
    assert par["heads"] == w.B * w.H and par["within_tolerance"], par
    assert par["o_max_abs"] < 1e-2 and par["lse_max_rel"] < 1e-6
    bad = o.clone()
    bad[0, 1, 17, 3] += 0.05
    _, par = bench.cpu_baseline(w, q, k, v, bad, lse)
    assert not par["within_tolerance"]
    assert par["o_max_abs"] == pytest.approx(
        abs(float(bad[0, 1, 17, 3]) - o_ref[0, 1, 17, 3]), rel=1e-6)


def test_int8_cache_roofline_mixes_the_two_matrix_peaks():
    """Half the INT8-cache FLOPs run on int8 matrix instructions (twice the
    16-bit rate), half on fp16 ones: the roof is 1 / (0.5/5033.2 + 0.5/2516.6)
    = 3355.5 TFLOP/s, and a launch at that roof's time reads frac 1."""
    w = WORKLOADS["int8_kv"]
    peak = 1.0 / (0.5 / 5033.2 + 0.5 / 2516.6)
    assert bench.matrix_peak(w) == pytest.approx(peak, abs=0.1)
    ms = w.flops / (peak * 1e12) * 1e3
    r = bench.roofline_of(w, ms, None)
    assert r["bound"] == "mfma" and r["frac"] == pytest.approx(1.0, abs=1e-3)
    assert bench.matrix_peak(WORKLOADS["headline"]) == 2516.6
