"""Host-side checks of bench.py that need no GPU: it refuses more than one
GPU, and its algorithmic work per stage and per step follows the stated
units (flops 6 N k H I + 2 N H E forward, 12 N k H I + 4 N H E backward;
bytes: x, the touched experts' weights and the outputs, each once)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import get  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name,gflop", [
    ("moe_top1_n4096_h768_e4", 45.93),
    ("dense_bf16_n16384_h2048_i6464", 1301.4),
    ("moe_top2_skew_n16384_h768_e8", 367.42),
    ("moe_decode_n32_h2048_e16", 1.109),
    ("dense_fp32_n100_h768_i2432", 1.1207),
])
def test_step_flops_match_the_stated_totals(name, gflop):
    w = get(name)
    assert abs(w.flops() / 1e9 - gflop) <= 1e-3 * gflop
    u = bench.stage_units(w)
    rows = w.N * (w.k if w.kind == "moe" else 1)
    assert u["gateup_gemm"][0] == 4.0 * rows * w.H * w.I
    assert u["down_gemm"][0] == 2.0 * rows * w.H * w.I
    assert sum(f for f, _ in u.values()) == pytest.approx(w.flops(), rel=1e-12)


def test_stage_bytes_count_each_tensor_once():
    w = get("moe_top1_n4096_h768_e4")
    el = w.elem_bytes()
    u = bench.stage_units(w)
    x, h = w.N * w.H * el, w.N * w.k * w.I * el
    wgu = 2 * w.E * w.I * w.H * el  # every expert is touched at this size
    assert u["gateup_gemm"][1] == x + wgu + h
    assert u["down_gemm"][1] == h + w.E * w.H * w.I * el + w.N * w.H * el


def test_backward_flops():
    for name in ("moe_top1_n4096_h768_e4", "dense_bf16_n16384_h2048_i6464"):
        w = get(name)
        rows = w.N * (w.k if w.kind == "moe" else 1)
        extra = 4.0 * w.N * w.H * w.E if w.kind == "moe" else 0.0
        assert bench.flops_bwd(w) == 12.0 * rows * w.H * w.I + extra
        u = bench.stage_units_bwd(w)
        gemm = sum(u[n][0] for n in ("dh_gemm", "dx_gemm", "dwgu_gemm", "dwd_gemm"))
        assert gemm == 12.0 * rows * w.H * w.I  # the recomputed g, u is not credited


def test_cpu_baseline_record_names_the_host():
    calls = []

    def run(n):
        calls.append(n)
        return 1.0 if n >= 1024 else 0.01

    n, times = bench.timed_sample(run, 4096, budget_s=6.0)
    assert n == 1024 and calls == [64, 256, 1024, 1024, 1024] and len(times) == 3
    rec = bench.baseline_record(n, times, 4096, "test")
    assert rec["value"] == pytest.approx(1024 / 1.0)
    assert rec["affinity_cpus"] == len(os.sched_getaffinity(0))
    assert rec["cores"] == rec["blas_threads"] >= 1
    assert rec["cpu_model"] and "median of 3" in rec["sample"]


def test_step_bytes_count_touched_weights_once():
    w = get("moe_decode_n32_h2048_e16")
    el = w.elem_bytes()
    assert bench.step_bytes(w, 16) == 2 * w.N * w.H * el + 3 * 16 * w.H * w.I * el + w.E * w.H * 4
    d = get("dense_bf16_n16384_h2048_i6464")
    assert bench.step_bytes(d, None) == 2 * d.N * d.H * 2 + 3 * d.H * d.I * 2


def test_default_workload_is_the_largest_configuration():
    from workloads.registry import WORKLOADS
    assert bench.DEFAULT_WORKLOAD == max(WORKLOADS.values(), key=lambda w: w.flops()).name
