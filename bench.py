"""Benchmark of the FP8 scaled linear layer on one MI355X.

Workload (the measured step): delayed-scaling FP8 linear fwd + bwd, tokens
4096, in 4096, out 4096, over 16 steps whose inputs are regenerated per step
from seed + step (X ~ N(0,1), W ~ N(0,0.02), dY ~ N(0,1e-4), bf16), all
resident in HBM before timing.  One step = the whole hot path:
  cast X -> E4M3 (+transpose, +amax), cast W -> E4M3 (+transpose, +amax),
  FWD GEMM (bf16 Y), cast dY -> E5M2 (+transpose, +amax), DGRAD GEMM (bf16
  dX), WGRAD GEMM (fp32 dW), amax-history update (len 16, max) for X, W, dY.
`value` = GEMM FLOPs of the step (3 x 2*4096^3) / measured step time, with
the K timed steps captured once into a HIP graph and replayed (the eager
per-call time is reported beside it as ms_per_step_eager).  The casts
max-accumulate their amax into slots that the history update clears after
reading them (fp8_cast_amax_acc, fp8_amax_history_update_reset); the same
step with overwriting casts, each zeroing its slot with a fill kernel
first, is reported as ms_per_step_overwrite_casts.

Also reported (same JSON line):
  roofline      -- the dominant kernel (the GEMMs), per-launch duration from
                   HIP events around R launches captured in a HIP graph, on
                   the stream the kernels run on;
  kernels       -- per-kernel throughput, warm (R launches back to back in one
                   graph, inputs left in the caches by the previous launch;
                   GEMM TFLOP/s, cast GB/s of algorithmic bytes) for this workload (also dY's cast with
                   stochastic rounding and the EWMA scale update), plus the forward
                   GEMM with its output quantised in the epilogue (E4M3,
                   transposed copy, amax) beside the unfused GEMM + cast;
  kernels_cold  -- the step's GEMMs, casts and amax timed cold: a 512 MiB
                   read evicts the 256 MB MALL before every launch (median
                   of single launches);
  rowwise       -- per-row (per-channel) scaling on the same shapes and data:
                   row-wise casts into both orientations and the three GEMMs
                   with per-row scales;
  blockwise     -- the block-wise path on 8192 tokens x 4096 in x 14336 out:
                   forward (1x128 activation tiles, 128x128 weight blocks)
                   and backward (dgrad, wgrad with token-axis tiles), with
                   binary32 block scales and with power-of-two ones, and
                   the row-wise path on the same shapes;
  cpu_baseline  -- the plain CPU oracle timed on a bounded sample of the
                   same step (rank 0, N = 1 only).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       [--no-blockwise] [--no-graph] [--kernel-reps R]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, TFLOP/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-blockwise", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--no-graph", action="store_true",
                    help="time the eager launches only (default: the K steps are captured "
                         "into one HIP graph and replayed)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the FP8 linear path here has no multi-GPU "
              "(sharded) mode; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from fp8_mixed_precision_linear_amd import datagen
    from fp8_mixed_precision_linear_amd import lib as L

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def d_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    T, DI, DO = 4096, 4096, 4096
    NSTEPS_DATA = 16
    t0 = time.time()
    data = []
    for t in range(NSTEPS_DATA):
        s = datagen.config2_step(t)
        data.append((d_bf16(s["x"]), d_bf16(s["w"]), d_bf16(s["dy"])))
    print(f"# generated 16 steps of inputs in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    u8 = dict(dtype=torch.uint8, device=dev)
    xq, xtq = torch.empty((T, DI), **u8), torch.empty((DI, T), **u8)
    wq, wtq = torch.empty((DI, DO), **u8), torch.empty((DO, DI), **u8)
    dyq, dytq = torch.empty((T, DO), **u8), torch.empty((DO, T), **u8)
    y = torch.empty((T, DO), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((T, DI), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((DI, DO), dtype=torch.float32, device=dev)
    hist = torch.zeros((3, 16), dtype=torch.float32, device=dev)
    scale = torch.ones(3, dtype=torch.float32, device=dev)
    sinv = torch.ones(3, dtype=torch.float32, device=dev)
    amax = torch.zeros(3, dtype=torch.float32, device=dev)

    # The casts max-accumulate their amax into the slots that the history
    # update reads and then clears (amax starts at 0), so a step needs no
    # zeroing kernel: 3 casts, 3 GEMMs, 2 history updates.
    def step(t):
        x, w, dyt = data[t % NSTEPS_DATA]
        L.fp8_cast_amax_acc(x, 0, scale[0:1], amax[0:1], y=xq, y_t=xtq)
        L.fp8_cast_amax_acc(w, 0, scale[1:2], amax[1:2], y=wq, y_t=wtq)
        L.fp8_scaled_gemm(xq, 0, 0, sinv[0:1], wtq, 0, 0, sinv[1:2], y)
        L.fp8_cast_amax_acc(dyt, 1, scale[2:3], amax[2:3], y=dyq, y_t=dytq)
        L.fp8_scaled_gemm(dyq, 1, 0, sinv[2:3], wq, 0, 0, sinv[1:2], dx)
        L.fp8_scaled_gemm(xtq, 0, 0, sinv[0:1], dytq, 1, 0, sinv[2:3], dw)
        L.fp8_amax_history_update_reset(hist[0:2], amax[0:2], 0, 0, 0, scale[0:2], sinv[0:2])
        L.fp8_amax_history_update_reset(hist[2:3], amax[2:3], 1, 0, 0, scale[2:3], sinv[2:3])

    # the same step with overwriting casts (each zeroes its amax slot with a
    # fill kernel first) and the plain history update, for comparison; timed
    # after the accumulating step's graph (it leaves the slots nonzero)
    def step_overwrite(t):
        x, w, dyt = data[t % NSTEPS_DATA]
        L.fp8_cast_e4m3(x, scale[0:1], y=xq, y_t=xtq, amax_out=amax[0:1])
        L.fp8_cast_e4m3(w, scale[1:2], y=wq, y_t=wtq, amax_out=amax[1:2])
        L.fp8_scaled_gemm(xq, 0, 0, sinv[0:1], wtq, 0, 0, sinv[1:2], y)
        L.fp8_cast_e5m2(dyt, scale[2:3], y=dyq, y_t=dytq, amax_out=amax[2:3])
        L.fp8_scaled_gemm(dyq, 1, 0, sinv[2:3], wq, 0, 0, sinv[1:2], dx)
        L.fp8_scaled_gemm(xtq, 0, 0, sinv[0:1], dytq, 1, 0, sinv[2:3], dw)
        L.fp8_amax_history_update(hist[0:2], amax[0:2], 0, 0, 0, scale[0:2], sinv[0:2])
        L.fp8_amax_history_update(hist[2:3], amax[2:3], 1, 0, 0, scale[2:3], sinv[2:3])

    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()

    # eager: one Python call per library entry point
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for t in range(args.steps):
        step(args.warmup + t)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step_eager = ev0.elapsed_time(ev1) / args.steps

    # graph: the same K steps captured once into a HIP graph and replayed
    # (no host launch cost; the GPU runs the identical kernel sequence)
    ms_step_graph = None
    ms_step_overwrite = None
    wall = None
    if not args.no_graph:
        g = capture(torch, lambda: [step(args.warmup + t) for t in range(args.steps)])
        g.replay()                      # warm-up replay (first launch uploads the graph)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        ev0.record(stream)
        g.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        ms_step_graph = ev0.elapsed_time(ev1) / args.steps
        del g
        g = capture(torch, lambda: [step_overwrite(args.warmup + t) for t in range(args.steps)])
        g.replay()
        torch.cuda.synchronize()
        ev0.record(stream)
        g.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        ms_step_overwrite = ev0.elapsed_time(ev1) / args.steps
        del g
    ms_step = ms_step_graph if ms_step_graph is not None else ms_step_eager
    gemm_flops = 3 * 2.0 * T * DI * DO
    value = gemm_flops / (ms_step * 1e-3) / 1e12

    # ---- per-kernel timing: R launches captured in a graph, one replay timed
    # with HIP events on the stream the kernels run on
    def time_launch(fn, reps):
        g = capture(torch, lambda: [fn() for _ in range(reps)])
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        del g
        return a.elapsed_time(b) / reps * 1e-3  # seconds per launch

    x0, w0, dy0 = data[0]
    R = args.kernel_reps
    k = {}
    k["gemm_fwd_tensor"] = time_launch(lambda: L.fp8_scaled_gemm(xq, 0, 0, sinv[0:1], wtq, 0, 0, sinv[1:2], y), R)
    k["gemm_dgrad_tensor"] = time_launch(lambda: L.fp8_scaled_gemm(dyq, 1, 0, sinv[2:3], wq, 0, 0, sinv[1:2], dx), R)
    k["gemm_wgrad_tensor"] = time_launch(lambda: L.fp8_scaled_gemm(xtq, 0, 0, sinv[0:1], dytq, 1, 0, sinv[2:3], dw), R)
    # the forward GEMM with its output quantised in the epilogue (E4M3 codes,
    # transposed copy, amax): the next layer's cast+transpose+amax fused in
    y8, y8t = torch.empty((T, DO), **u8), torch.empty((DO, T), **u8)
    am8 = torch.zeros(1, dtype=torch.float32, device=dev)
    k["gemm_fwd_tensor_fp8out"] = time_launch(
        lambda: L.fp8_scaled_gemm(xq, 0, 0, sinv[0:1], wtq, 0, 0, sinv[1:2], y8, d_amax=am8,
                                  d_scale=scale[0:1], d_fmt=0, D_t=y8t), R)
    k["cast_transpose_amax_e4m3"] = time_launch(lambda: L.fp8_cast_e4m3(x0, scale[0:1], y=xq, y_t=xtq, amax_out=amax[0:1]), R)
    k["cast_transpose_amax_acc_e4m3"] = time_launch(lambda: L.fp8_cast_amax_acc(x0, 0, scale[0:1], amax[0:1], y=xq, y_t=xtq), R)
    k["cast_transpose_amax_e5m2"] = time_launch(lambda: L.fp8_cast_e5m2(dy0, scale[2:3], y=dyq, y_t=dytq, amax_out=amax[2:3]), R)
    k["cast_transpose_amax_e5m2_sr"] = time_launch(
        lambda: L.fp8_cast_sr(dy0, 1, scale[2:3], 1234, 0, y=dyq, y_t=dytq, amax_out=amax[2:3]), R)
    k["cast_e4m3"] = time_launch(lambda: L.fp8_cast_e4m3(x0, scale[0:1], y=xq), R)
    k["amax"] = time_launch(lambda: L.fp8_amax(x0, amax[0:1]), R)
    k["history_update"] = time_launch(lambda: L.fp8_amax_history_update(hist[0:2], amax[0:2], 0, 0, 0, scale[0:2], sinv[0:2]), R)
    ewma = torch.zeros(3, dtype=torch.float32, device=dev)
    k["ewma_update"] = time_launch(lambda: L.fp8_amax_ewma_update(ewma, amax, 0.9, 0, 0, scale, sinv), R)
    nel = T * DI
    kernels = {
        "gemm_fwd_tensor": {"tflops": 2.0 * T * DI * DO / k["gemm_fwd_tensor"] / 1e12, "us": k["gemm_fwd_tensor"] * 1e6},
        "gemm_dgrad_tensor": {"tflops": 2.0 * T * DI * DO / k["gemm_dgrad_tensor"] / 1e12, "us": k["gemm_dgrad_tensor"] * 1e6},
        "gemm_wgrad_tensor": {"tflops": 2.0 * T * DI * DO / k["gemm_wgrad_tensor"] / 1e12, "us": k["gemm_wgrad_tensor"] * 1e6},
        "gemm_fwd_tensor_fp8out": {"tflops": 2.0 * T * DI * DO / k["gemm_fwd_tensor_fp8out"] / 1e12,
                                   "us": k["gemm_fwd_tensor_fp8out"] * 1e6,
                                   "us_unfused_equivalent": (k["gemm_fwd_tensor"] + k["cast_transpose_amax_e4m3"]) * 1e6},
        "cast_transpose_amax_e4m3": {"gbs": 4.0 * nel / k["cast_transpose_amax_e4m3"] / 1e9, "us": k["cast_transpose_amax_e4m3"] * 1e6},
        "cast_transpose_amax_acc_e4m3": {"gbs": 4.0 * nel / k["cast_transpose_amax_acc_e4m3"] / 1e9,
                                         "us": k["cast_transpose_amax_acc_e4m3"] * 1e6},
        "cast_transpose_amax_e5m2": {"gbs": 4.0 * nel / k["cast_transpose_amax_e5m2"] / 1e9, "us": k["cast_transpose_amax_e5m2"] * 1e6},
        "cast_transpose_amax_e5m2_sr": {"gbs": 4.0 * nel / k["cast_transpose_amax_e5m2_sr"] / 1e9,
                                        "us": k["cast_transpose_amax_e5m2_sr"] * 1e6},
        "cast_e4m3": {"gbs": 3.0 * nel / k["cast_e4m3"] / 1e9, "us": k["cast_e4m3"] * 1e6},
        "amax": {"gbs": 2.0 * nel / k["amax"] / 1e9, "us": k["amax"] * 1e6},
        "history_update": {"us": k["history_update"] * 1e6},
        "ewma_update": {"us": k["ewma_update"] * 1e6},
    }
    # ---- row-wise (per-channel) scaling on the same shapes: each operand
    # cast once into both orientations (row scales, column scales), the
    # three GEMMs with per-row scales applied in the epilogue
    f32 = dict(dtype=torch.float32, device=dev)
    sxr, sxc = torch.empty(T, **f32), torch.empty(DI, **f32)
    swr, swc = torch.empty(DI, **f32), torch.empty(DO, **f32)
    sdr, sdc = torch.empty(T, **f32), torch.empty(DO, **f32)
    k["cast_rowwise_x"] = time_launch(lambda: L.fp8_cast_rowwise(x0, 0, xq, sxr, xtq, sxc), R)
    k["cast_rowwise_w"] = time_launch(lambda: L.fp8_cast_rowwise(w0, 0, wq, swr, wtq, swc), R)
    k["cast_rowwise_dy"] = time_launch(lambda: L.fp8_cast_rowwise(dy0, 1, dyq, sdr, dytq, sdc), R)
    k["gemm_fwd_rowwise"] = time_launch(lambda: L.fp8_scaled_gemm(xq, 0, 5, sxr, wtq, 0, 5, swc, y), R)
    k["gemm_dgrad_rowwise"] = time_launch(lambda: L.fp8_scaled_gemm(dyq, 1, 5, sdr, wq, 0, 5, swr, dx), R)
    k["gemm_wgrad_rowwise"] = time_launch(lambda: L.fp8_scaled_gemm(xtq, 0, 5, sxc, dytq, 1, 5, sdc, dw), R)
    rowwise = rowwise_summary(k, T, DI, DO, "row-wise fwd+dgrad+wgrad, tokens 4096, in 4096, out 4096 "
                                           "(delayed-scaling workload data, step 0)")
    g_avg = (k["gemm_fwd_tensor"] + k["gemm_dgrad_tensor"] + k["gemm_wgrad_tensor"]) / 3
    g_ach = 2.0 * T * DI * DO / g_avg / 1e12
    roofline = {"bound": "mfma",
                "kernel": "k_gemm_big, per-tensor scales, 4096^3 (fwd/dgrad/wgrad average)",
                "achieved": round(g_ach, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(g_ach / FP8_PEAK_TFLOPS, 4), "traffic": gemm_traffic()}

    # ---- cold timings: before every timed launch a 512 MiB read evicts the
    # 256 MB last-level cache (MALL) with clean lines, so inputs come from
    # HBM and no dirty victims are written back during the timed kernel; each
    # launch is bracketed by its own HIP events on the stream (median of the
    # reps; the brackets include the dispatch of that one launch)
    flush = torch.zeros(256 << 20, dtype=torch.bfloat16, device=dev)
    flush_amax = torch.zeros(1, dtype=torch.float32, device=dev)
    L.fp8_amax(flush, flush_amax)
    torch.cuda.synchronize()

    def time_cold(fn, reps):
        evs = []
        for i in range(reps):
            L.fp8_amax(flush, flush_amax)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in evs)
        return ts[len(ts) // 2] * 1e-3   # seconds

    kc = {}
    kc["gemm_fwd_tensor"] = time_cold(lambda: L.fp8_scaled_gemm(xq, 0, 0, sinv[0:1], wtq, 0, 0, sinv[1:2], y), R)
    kc["gemm_dgrad_tensor"] = time_cold(lambda: L.fp8_scaled_gemm(dyq, 1, 0, sinv[2:3], wq, 0, 0, sinv[1:2], dx), R)
    kc["gemm_wgrad_tensor"] = time_cold(lambda: L.fp8_scaled_gemm(xtq, 0, 0, sinv[0:1], dytq, 1, 0, sinv[2:3], dw), R)
    kc["cast_transpose_amax_acc_e4m3"] = time_cold(lambda: L.fp8_cast_amax_acc(x0, 0, scale[0:1], amax[0:1], y=xq, y_t=xtq), R)
    kc["cast_transpose_amax_acc_e5m2"] = time_cold(lambda: L.fp8_cast_amax_acc(dy0, 1, scale[2:3], amax[2:3], y=dyq, y_t=dytq), R)
    kc["cast_e4m3"] = time_cold(lambda: L.fp8_cast_e4m3(x0, scale[0:1], y=xq), R)
    kc["amax"] = time_cold(lambda: L.fp8_amax(x0, amax[0:1]), R)
    del flush
    kernels_cold = {"note": "MALL evicted (512 MiB read) before every timed launch; median of "
                            f"{R} single launches, each bracketed by HIP events"}
    for n in ("gemm_fwd_tensor", "gemm_dgrad_tensor", "gemm_wgrad_tensor"):
        kernels_cold[n] = {"tflops": round(2.0 * T * DI * DO / kc[n] / 1e12, 2), "us": round(kc[n] * 1e6, 2)}
    for n, bpe in (("cast_transpose_amax_acc_e4m3", 4.0), ("cast_transpose_amax_acc_e5m2", 4.0),
                   ("cast_e4m3", 3.0), ("amax", 2.0)):
        kernels_cold[n] = {"gbs": round(bpe * nel / kc[n] / 1e9, 2), "us": round(kc[n] * 1e6, 2),
                           "pct_hbm_peak": round(100 * bpe * nel / kc[n] / 1e9 / HBM_PEAK_GBS, 2)}

    # ---- block-wise path at 8192 x 4096 x 14336
    blockwise = None
    if not args.no_blockwise:
        blockwise = bench_blockwise(torch, L, datagen, dev, stream, d_bf16, time_launch, R)

    result = {
        "metric": "FP8 scaled-GEMM TFLOP/s (fwd+dgrad+wgrad, % FP8 peak) + cast GB/s",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "launch": "hip_graph" if ms_step_graph is not None else "eager",
        "ms_per_step_eager": round(ms_step_eager, 4),
        "ms_per_step_overwrite_casts": (round(ms_step_overwrite, 4)
                                        if ms_step_overwrite is not None else None),
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8-e4m3/e5m2 (fp32 accumulate)",
        "data": "synthetic (seeded numpy PCG64, bf16)",
        "config": {"workload": "delayed-scaling FP8 linear fwd+dgrad+wgrad, tokens 4096, in 4096, "
                               "out 4096, amax history 16, inputs regenerated per step (16 steps)",
                   "global_batch": T, "seq_len": None, "parallelism": "none (1 GPU)"},
        "wall_s_timed": round(wall, 4) if wall is not None else None,
        "pct_fp8_peak": round(100 * value / FP8_PEAK_TFLOPS, 2),
        "roofline": roofline,
        "kernels": {n: {kk: round(vv, 2) for kk, vv in d.items()} for n, d in kernels.items()},
        "kernels_cold": kernels_cold,
    }
    result["rowwise"] = rowwise
    if blockwise is not None:
        result["blockwise"] = blockwise
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(gemm_flops)
    print(json.dumps(result), flush=True)


def bench_blockwise(torch, L, datagen, dev, stream, d_bf16, time_launch, R):
    T, DI, DO = 8192, 4096, 14336
    t0 = time.time()
    c3 = datagen.config3()
    x, w = d_bf16(c3["x"]), d_bf16(c3["w"])
    dy = d_bf16(datagen.config4_dy(c3["rng"]))
    print(f"# generated block-wise inputs in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    xq, sx = torch.empty((T, DI), **u8), torch.empty((DI // 128, T), **f32)
    xtq, sxt = torch.empty((DI, T), **u8), torch.empty((T // 128, DI), **f32)
    wq, sw = torch.empty((DI, DO), **u8), torch.empty((DO // 128, DI // 128), **f32)
    wtq, swt = torch.empty((DO, DI), **u8), torch.empty((DI // 128, DO // 128), **f32)
    dyq, sdy = torch.empty((T, DO), **u8), torch.empty((DO // 128, T), **f32)
    dytq, sdyt = torch.empty((DO, T), **u8), torch.empty((T // 128, DO), **f32)
    y = torch.empty((T, DO), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((T, DI), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((DI, DO), **f32)
    k = {}
    k["cast_block_x_dual"] = time_launch(lambda: L.fp8_cast_block(x, 0, 1, xq, sx, xtq, sxt), R)
    k["cast_block_x_1x128"] = time_launch(lambda: L.fp8_cast_block(x, 0, 1, xq, sx), R)
    k["cast_block_w_128x128_both"] = time_launch(lambda: L.fp8_cast_block(w, 0, 2, wq, sw, wtq, swt), R)
    k["cast_block_dy_dual"] = time_launch(lambda: L.fp8_cast_block(dy, 1, 1, dyq, sdy, dytq, sdyt), R)
    k["gemm_fwd_block"] = time_launch(lambda: L.fp8_scaled_gemm(xq, 0, 1, sx, wtq, 0, 2, swt, y), R)
    k["gemm_dgrad_block"] = time_launch(lambda: L.fp8_scaled_gemm(dyq, 1, 1, sdy, wq, 0, 2, sw, dx), R)
    k["gemm_wgrad_block"] = time_launch(lambda: L.fp8_scaled_gemm(xtq, 0, 1, sxt, dytq, 1, 1, sdyt, dw), R)
    # the same path with power-of-two (exponent-bias) block scales: the GEMMs
    # apply them inside the E8M0-scaled matrix instruction
    k["cast_block_pow2_x_dual"] = time_launch(lambda: L.fp8_cast_block_pow2(x, 0, 1, xq, sx, xtq, sxt), R)
    k["cast_block_pow2_w_128x128_both"] = time_launch(lambda: L.fp8_cast_block_pow2(w, 0, 2, wq, sw, wtq, swt), R)
    k["cast_block_pow2_dy_dual"] = time_launch(lambda: L.fp8_cast_block_pow2(dy, 1, 1, dyq, sdy, dytq, sdyt), R)
    k["gemm_fwd_block_pow2"] = time_launch(lambda: L.fp8_scaled_gemm(xq, 0, 3, sx, wtq, 0, 4, swt, y), R)
    k["gemm_dgrad_block_pow2"] = time_launch(lambda: L.fp8_scaled_gemm(dyq, 1, 3, sdy, wq, 0, 4, sw, dx), R)
    k["gemm_wgrad_block_pow2"] = time_launch(lambda: L.fp8_scaled_gemm(xtq, 0, 3, sxt, dytq, 1, 3, sdyt, dw), R)
    fl = 2.0 * T * DI * DO
    out = {"workload": "block-wise fwd (X 8192x4096 Student-t 1x128, W 4096x14336 128x128) + "
                       "bwd (dY 8192x14336 1x128 dual orientation; dgrad, wgrad)"}
    for n in ("gemm_fwd_block", "gemm_dgrad_block", "gemm_wgrad_block", "gemm_fwd_block_pow2",
              "gemm_dgrad_block_pow2", "gemm_wgrad_block_pow2"):
        out[n] = {"tflops": round(fl / k[n] / 1e12, 2), "us": round(k[n] * 1e6, 1),
                  "pct_fp8_peak": round(100 * fl / k[n] / 1e12 / FP8_PEAK_TFLOPS, 2)}
    bytes_ = {"cast_block_x_dual": T * DI * (4 + 8 / 128), "cast_block_x_1x128": T * DI * (3 + 4 / 128),
              "cast_block_w_128x128_both": DI * DO * 4.0, "cast_block_dy_dual": T * DO * (4 + 8 / 128),
              "cast_block_pow2_x_dual": T * DI * (4 + 8 / 128),
              "cast_block_pow2_w_128x128_both": DI * DO * 4.0,
              "cast_block_pow2_dy_dual": T * DO * (4 + 8 / 128)}
    for n, b in bytes_.items():
        out[n] = {"gbs": round(b / k[n] / 1e9, 1), "us": round(k[n] * 1e6, 1),
                  "pct_hbm_peak": round(100 * b / k[n] / 1e9 / HBM_PEAK_GBS, 2)}
    tot = (k["cast_block_x_dual"] + k["cast_block_w_128x128_both"] + k["cast_block_dy_dual"]
           + k["gemm_fwd_block"] + k["gemm_dgrad_block"] + k["gemm_wgrad_block"])
    out["fwd_bwd_tflops_incl_casts"] = round(3 * fl / tot / 1e12, 2)
    out["fwd_bwd_ms"] = round(tot * 1e3, 3)
    tot2 = (k["cast_block_pow2_x_dual"] + k["cast_block_pow2_w_128x128_both"]
            + k["cast_block_pow2_dy_dual"] + k["gemm_fwd_block_pow2"] + k["gemm_dgrad_block_pow2"]
            + k["gemm_wgrad_block_pow2"])
    out["fwd_bwd_tflops_incl_casts_pow2"] = round(3 * fl / tot2 / 1e12, 2)
    out["fwd_bwd_ms_pow2"] = round(tot2 * 1e3, 3)
    # row-wise scaling on the same shapes and data
    sxr, sxc = torch.empty(T, **f32), torch.empty(DI, **f32)
    swr, swc = torch.empty(DI, **f32), torch.empty(DO, **f32)
    sdr, sdc = torch.empty(T, **f32), torch.empty(DO, **f32)
    r = {}
    r["cast_rowwise_x"] = time_launch(lambda: L.fp8_cast_rowwise(x, 0, xq, sxr, xtq, sxc), R)
    r["cast_rowwise_w"] = time_launch(lambda: L.fp8_cast_rowwise(w, 0, wq, swr, wtq, swc), R)
    r["cast_rowwise_dy"] = time_launch(lambda: L.fp8_cast_rowwise(dy, 1, dyq, sdr, dytq, sdc), R)
    r["gemm_fwd_rowwise"] = time_launch(lambda: L.fp8_scaled_gemm(xq, 0, 5, sxr, wtq, 0, 5, swc, y), R)
    r["gemm_dgrad_rowwise"] = time_launch(lambda: L.fp8_scaled_gemm(dyq, 1, 5, sdr, wq, 0, 5, swr, dx), R)
    r["gemm_wgrad_rowwise"] = time_launch(lambda: L.fp8_scaled_gemm(xtq, 0, 5, sxc, dytq, 1, 5, sdc, dw), R)
    out["rowwise"] = rowwise_summary(r, T, DI, DO, "row-wise on the same shapes and data")
    return out


def rowwise_summary(k, T, DI, DO, workload):
    """Row-wise path: GEMM TFLOP/s, cast GB/s of algorithmic bytes (bf16 read
    once, both FP8 orientations written once, row and column scales), and
    the whole fwd+bwd including the three casts."""
    fl = 2.0 * T * DI * DO
    out = {"workload": workload}
    for n in ("gemm_fwd_rowwise", "gemm_dgrad_rowwise", "gemm_wgrad_rowwise"):
        out[n] = {"tflops": round(fl / k[n] / 1e12, 2), "us": round(k[n] * 1e6, 1),
                  "pct_fp8_peak": round(100 * fl / k[n] / 1e12 / FP8_PEAK_TFLOPS, 2)}
    shapes = {"cast_rowwise_x": (T, DI), "cast_rowwise_w": (DI, DO), "cast_rowwise_dy": (T, DO)}
    for n, (a, b) in shapes.items():
        by = a * b * 4.0 + 4.0 * (a + b)
        out[n] = {"gbs": round(by / k[n] / 1e9, 1), "us": round(k[n] * 1e6, 1),
                  "pct_hbm_peak": round(100 * by / k[n] / 1e9 / HBM_PEAK_GBS, 2)}
    tot = sum(k[n] for n in list(shapes) + ["gemm_fwd_rowwise", "gemm_dgrad_rowwise",
                                            "gemm_wgrad_rowwise"])
    out["fwd_bwd_tflops_incl_casts"] = round(3 * fl / tot / 1e12, 2)
    out["fwd_bwd_ms"] = round(tot * 1e3, 3)
    return out


def gemm_traffic():
    """HBM bytes per launch of the per-tensor 4096^3 GEMM (average of fwd,
    dgrad, wgrad) from the committed counter summary, or None when the
    kernel sources changed after the counters were taken."""
    path = os.path.join(ROOT, "profiles", "gemm_tensor4096_traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
        from fp8_mixed_precision_linear_amd.traffic_probe import sources_sha256
        if t.get("sources_sha256") != sources_sha256():
            return None
        k = t["kernels"]
        names = ("gemm_fwd_tensor", "gemm_dgrad_tensor", "gemm_wgrad_tensor")
        return round(sum(k[n]["traffic_bytes"] for n in names) / 3)
    except (OSError, KeyError, ValueError):
        return None


def capture(torch, fn):
    """Capture fn's launches into a HIP graph (torch makes its capture stream
    the current stream, which is the stream the binding passes to the
    library)."""
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def cpu_baseline(gemm_flops):
    """The oracle, as it stands, on a bounded sample of one step: the three
    casts (+amax) of one step at full size, and the three GEMMs (exact and
    FP32-accumulated) on 64 sampled output rows each, extrapolated to the
    full 4096 rows."""
    from fp8_mixed_precision_linear_amd import datagen
    from oracle import oracle as O
    s = datagen.config2_step(0)
    t0 = time.perf_counter()
    ax, aw, ad = O.amax_parallel(s["x"]), O.amax_parallel(s["w"]), O.amax_parallel(s["dy"])
    xq = O.cast(s["x"], 1.0, 0)
    wq = O.cast(s["w"], 1.0, 0)
    dq = O.cast(s["dy"], 1.0, 1)
    t_cast = time.perf_counter() - t0
    rows = np.arange(64, dtype=np.int64)
    one = np.ones(1, np.float32)
    wt = np.ascontiguousarray(wq.T)
    t1 = time.perf_counter()
    O.gemm(xq, 0, 0, one, wt, 0, 0, one, ms=rows)                 # fwd
    O.gemm(dq, 1, 0, one, wq, 0, 0, one, ms=rows)                 # dgrad
    O.gemm(np.ascontiguousarray(xq.T), 0, 0, one, np.ascontiguousarray(dq.T), 1, 0, one, ms=rows)
    t_gemm = (time.perf_counter() - t1) * (4096 / 64)
    t_step = t_cast + t_gemm
    return {"value": round(gemm_flops / t_step / 1e12, 6), "unit": "TFLOP/s", "cores": O.nthreads(),
            "kind": "oracle",
            "sample": "one delayed-scaling step (4096^3): casts + amax at full size "
                      f"({t_cast:.2f}s), the three GEMMs on 64 of 4096 output rows "
                      f"({t_gemm * 64 / 4096:.2f}s), extrapolated to all rows",
            "step_s_extrapolated": round(t_step, 2)}


if __name__ == "__main__":
    main()
