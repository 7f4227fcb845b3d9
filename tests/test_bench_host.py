"""Host-side checks of bench.py (CPU only): the one-GPU guard, the launch
plan of the transformer-block step and the per-pass aggregation of its
timings.

The step is the FP8 linear set of a decoder block, [MPG] "Mixed precision
in real architectures > Standard transformer (decoder-only)": QKV, output
projection and the gated FFN (gate / up share one input), hidden 8192, FFN
28672, 8192 tokens, forward + dgrad + wgrad of each linear, once per scaling
mode.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

T, H, F = 8192, 8192, 28672
LINEARS = {"qkv": (H, 10240), "o": (H, H), "gate": (H, F), "up": (H, F), "down": (F, H)}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120,
                       env={**os.environ, "WORLD_SIZE": "1"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_step_plan_counts_and_flops():
    plan = bench.c5_plan()
    assert len(plan) == 60
    gemms = [p for p in plan if p[1] == "gemm"]
    assert len(gemms) == 30
    # every linear runs FWD, DGRAD and WGRAD in each mode, 2 T d_in d_out FLOPs each
    for mode in ("delayed", "block"):
        for n, (di, do) in LINEARS.items():
            for op in ("fwd", "dgrad", "wgrad"):
                (w,) = [w for lab, k, w in gemms if lab == f"{mode} {op} {n}"]
                assert w == 2.0 * T * di * do
    total = sum(w for _, _, w in gemms)
    per_mode = 3 * sum(2.0 * T * di * do for di, do in LINEARS.values())
    assert total == 2 * per_mode
    assert abs(per_mode / 1e12 - 42.06) < 0.01
    # gate and up share one activation: four X casts per mode, five W and dY casts
    for mode in ("delayed", "block"):
        for kind, count in (("cast X", 4), ("cast W", 5), ("cast dY", 5)):
            assert len([1 for lab, _, _ in plan if lab.startswith(f"{mode} {kind} ")]) == count


def test_step_plan_cast_bytes():
    plan = {lab: w for lab, _, w in bench.c5_plan()}
    # per-tensor cast + transpose: 2 B read, 1 + 1 B written per element
    assert plan["delayed cast X qkv"] == 4.0 * T * H
    assert plan["delayed cast W down"] == 4.0 * F * H
    # block dual cast: the same plus one binary32 scale per 128 elements and orientation
    assert plan["block cast dY gate"] == pytest.approx(T * F * (4 + 8 / 128))
    # 128 x 128 weight blocks: one scale per block for each copy
    assert plan["block cast W o"] == pytest.approx(H * H * (4 + 8 / 16384))


def test_summary_aggregates():
    plan = bench.c5_plan()
    # synthetic timings: every GEMM at exactly 2.5 PFLOP/s, every cast at 5 TB/s
    timed = []
    for lab, kind, w in plan:
        sec = w / 2.5e15 if kind == "gemm" else (w / 5e12 if kind == "cast" else 2e-6)
        timed.append((lab, kind, w, sec))
    s = bench.c5_summary(timed)
    for mode in ("delayed", "block"):
        assert s[mode]["gemm_tflops"] == pytest.approx(2500.0, abs=0.1)
        assert s[mode]["cast_gbs"] == pytest.approx(5000.0, abs=0.1)
        assert s[mode]["gemm_pct_fp8_peak"] == pytest.approx(50.0, abs=0.01)
    assert s["delayed"]["other_ms"] == pytest.approx(0.004)
    k = s["gemm_kernels"]
    assert set(k) == set(bench.C5_KERNEL)
    for cls, e in k.items():
        assert e["launches"] == 5
        assert e["kernel"] == bench.C5_KERNEL[cls]
        assert e["tflops"] == pytest.approx(2500.0, abs=0.1)
    # the WGRAD kernel's FLOPs per launch: the five linears' average
    avg = sum(2.0 * T * di * do for di, do in LINEARS.values()) / 5
    assert k["block wgrad"]["flop_per_launch"] == pytest.approx(avg)
