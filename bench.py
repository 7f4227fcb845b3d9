"""Benchmark of the FP8 scaled linear layer on one MI355X.

Workload (the measured step): the transformer-block FP8 linear set at
hidden 8192, FFN 28672, 8192 tokens -- QKV 8192 -> 10240, O 8192 -> 8192,
gate and up 8192 -> 28672 each (one shared activation), down 28672 -> 8192 --
forward, dgrad and wgrad of every linear, once in per-tensor delayed
scaling and once in block-wise scaling.  One step runs both passes, so it
covers the whole hot path: amax fused into the casts, scales from the amax
histories, saturating RNE casts with fused transposes (per-tensor and
block-wise), and the FWD / DGRAD / WGRAD GEMMs with FP32 accumulation,
block-scale promotion and the dequantising epilogue.

  delayed pass: per linear (forward order) cast X and W (E4M3, both
    orientations, amax max-accumulated into the tensor's slot), FWD GEMM
    (bf16 Y); per linear (backward order) cast dY (E5M2), DGRAD (bf16 dX),
    WGRAD (fp32 dW); then the amax-history update (length 16, max) of all
    14 tensors (two calls: E4M3 and E5M2), which also clears the slots;
  block pass: the same with block-wise casts (X and dY 1x128 tiles in both
    orientations, W 128x128 blocks with the transposed copy) and block
    scales promoted per 128-wide K block in the GEMMs.

Inputs are synthetic (seeded numpy PCG64, bf16) and resident in HBM before
timing; warm-up steps fill the amax histories first.  `value` = GEMM FLOPs
of one step (2 x 42.06 TFLOP) / measured step time, the K timed steps
captured once into a HIP graph and replayed.

Also reported (same JSON line):
  c5            -- per pass and per linear: every launch of one eager step
                   bracketed by HIP events on the library's stream (GEMM
                   TFLOP/s, cast GB/s of algorithmic bytes);
  roofline      -- the dominant kernel of the step (the GEMM kernel with the
                   largest share of the step), achieved = its FLOPs per
                   launch / its average launch duration from those events;
                   traffic from the committed counter summary while the
                   kernel sources are unchanged;
  delayed4096, kernels, kernels_cold, rowwise, blockwise -- the smaller
                   workloads (delayed-scaling fwd+bwd at 4096^3; per-kernel
                   throughput warm and with the 256 MB last-level cache
                   evicted before every launch; per-row scaling; the
                   block-wise path at 8192 x 4096 x 14336);
  cpu_baseline  -- the plain CPU oracle timed on a bounded sample of the step
                   (rank 0, N = 1 only).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       [--no-extras] [--kernel-reps R]
       python bench.py --traffic-run            (under rocprofv3 --pmc)
       python bench.py --traffic-summarize DIR OUT.json
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import subprocess
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, TFLOP/s
C5_ORDER = ["qkv", "o", "gate", "up", "down"]
C5_X = {"qkv": "qkv", "o": "o", "gate": "gate", "up": "gate", "down": "down"}
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "gemm_c5_traffic.json")
TRAFFIC_SOURCES = ("csrc/gemm_big_kernel.h", "csrc/gemm_big.hip", "csrc/gemm_w4_kernel.h",
                   "csrc/gemm_w4.hip", "csrc/fp8_device.h", "build.py")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the headline step (no 4096^3 / 8192x4096x14336 extras)")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--traffic-run", action="store_true",
                    help="run the step's GEMMs and a copy of known size (for rocprofv3 --pmc)")
    ap.add_argument("--traffic-summarize", nargs=2, metavar=("DIR", "OUT"))
    return ap.parse_args()


# ----------------------------------------------------------------------------
# the transformer-block linear set
# ----------------------------------------------------------------------------
class C5Set:
    """Device tensors of the five linears (inputs, FP8 operands in both
    orientations, outputs, delayed-scaling state and block scales) and the
    launches of one step, as (label, kind, work, fn) with kind gemm (work =
    FLOPs) or cast / state (work = algorithmic bytes)."""

    def __init__(self, torch, L, datagen, dev):
        self.torch, self.L = torch, L
        bf = dict(dtype=torch.bfloat16, device=dev)
        u8 = dict(dtype=torch.uint8, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)

        def d_bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

        self.shapes = {n: datagen.C5_LINEARS[n] for n in C5_ORDER}
        T = 8192
        self.T = T
        t0 = time.time()
        self.x, self.w, self.dy = {}, {}, {}
        for n in C5_ORDER:
            parts = ("x", "w", "dy") if C5_X[n] == n else ("w", "dy")
            d = datagen.config5_linear(n, parts=parts)
            if "x" in d:
                self.x[n] = d_bf16(d["x"])
            self.w[n] = d_bf16(d["w"])
            self.dy[n] = d_bf16(d["dy"])
            del d
        self.gen_s = time.time() - t0
        # FP8 operands (shared by both passes), outputs
        self.xq, self.xtq = {}, {}
        for n in self.x:
            di = self.shapes[n][0]
            self.xq[n], self.xtq[n] = torch.empty((T, di), **u8), torch.empty((di, T), **u8)
        self.wq, self.wtq, self.dyq, self.dytq, self.y, self.dx, self.dw = ({} for _ in range(7))
        for n in C5_ORDER:
            di, do = self.shapes[n]
            self.wq[n], self.wtq[n] = torch.empty((di, do), **u8), torch.empty((do, di), **u8)
            self.dyq[n], self.dytq[n] = torch.empty((T, do), **u8), torch.empty((do, T), **u8)
            self.y[n] = torch.empty((T, do), **bf)
            self.dx[n] = torch.empty((T, di), **bf)
            self.dw[n] = torch.empty((di, do), **f32)
        # delayed-scaling state: E4M3 tensors first (X of 4 inputs, W of 5
        # linears), then E5M2 (dY of 5 linears); one amax slot per tensor
        xs = list(self.x)
        self.slot = {("x", n): i for i, n in enumerate(xs)}
        for i, n in enumerate(C5_ORDER):
            self.slot[("w", n)] = len(xs) + i
            self.slot[("dy", n)] = len(xs) + len(C5_ORDER) + i
        self.n_e4m3 = len(xs) + len(C5_ORDER)
        nt = self.n_e4m3 + len(C5_ORDER)
        self.hist = torch.zeros((nt, 16), **f32)
        self.scale = torch.ones(nt, **f32)
        self.sinv = torch.ones(nt, **f32)
        self.amax = torch.zeros(nt, **f32)
        # block scales
        self.sx, self.sxt, self.sw, self.swt, self.sd, self.sdt = ({} for _ in range(6))
        for n in xs:
            di = self.shapes[n][0]
            self.sx[n] = torch.empty((di // 128, T), **f32)
            self.sxt[n] = torch.empty((T // 128, di), **f32)
        for n in C5_ORDER:
            di, do = self.shapes[n]
            self.sw[n] = torch.empty((do // 128, di // 128), **f32)
            self.swt[n] = torch.empty((di // 128, do // 128), **f32)
            self.sd[n] = torch.empty((do // 128, T), **f32)
            self.sdt[n] = torch.empty((T // 128, do), **f32)
        self.ops = {"delayed": self._delayed_ops(), "block": self._block_ops()}
        assert [op[:3] for m in ("delayed", "block") for op in self.ops[m]] == c5_plan(T)

    def flops_per_pass(self):
        return sum(3 * 2.0 * self.T * di * do for di, do in self.shapes.values())

    def _delayed_ops(self):
        L, T, s, si, am = self.L, self.T, self.scale, self.sinv, self.amax
        ops = []

        def sl(key):
            i = self.slot[key]
            return i, i + 1

        for n in C5_ORDER:
            di, do = self.shapes[n]
            xn = C5_X[n]
            xa, xb = sl(("x", xn))
            wa, wb = sl(("w", n))
            if xn == n:
                ops.append((f"delayed cast X {n}", "cast", 4.0 * T * di,
                            lambda xn=xn, xa=xa, xb=xb: L.fp8_cast_amax_acc(
                                self.x[xn], 0, s[xa:xb], am[xa:xb], y=self.xq[xn], y_t=self.xtq[xn])))
            ops.append((f"delayed cast W {n}", "cast", 4.0 * di * do,
                        lambda n=n, wa=wa, wb=wb: L.fp8_cast_amax_acc(
                            self.w[n], 0, s[wa:wb], am[wa:wb], y=self.wq[n], y_t=self.wtq[n])))
            ops.append((f"delayed fwd {n}", "gemm", 2.0 * T * di * do,
                        lambda n=n, xn=xn, xa=xa, xb=xb, wa=wa, wb=wb: L.fp8_scaled_gemm(
                            self.xq[xn], 0, 0, si[xa:xb], self.wtq[n], 0, 0, si[wa:wb], self.y[n])))
        for n in reversed(C5_ORDER):
            di, do = self.shapes[n]
            xn = C5_X[n]
            xa, xb = sl(("x", xn))
            wa, wb = sl(("w", n))
            da, db = sl(("dy", n))
            ops.append((f"delayed cast dY {n}", "cast", 4.0 * T * do,
                        lambda n=n, da=da, db=db: L.fp8_cast_amax_acc(
                            self.dy[n], 1, s[da:db], am[da:db], y=self.dyq[n], y_t=self.dytq[n])))
            ops.append((f"delayed dgrad {n}", "gemm", 2.0 * T * di * do,
                        lambda n=n, wa=wa, wb=wb, da=da, db=db: L.fp8_scaled_gemm(
                            self.dyq[n], 1, 0, si[da:db], self.wq[n], 0, 0, si[wa:wb], self.dx[n])))
            ops.append((f"delayed wgrad {n}", "gemm", 2.0 * T * di * do,
                        lambda n=n, xn=xn, xa=xa, xb=xb, da=da, db=db: L.fp8_scaled_gemm(
                            self.xtq[xn], 0, 0, si[xa:xb], self.dytq[n], 1, 0, si[da:db], self.dw[n])))
        e = self.n_e4m3
        ops.append(("delayed history E4M3", "state", 8.0 * 16 * e,
                    lambda: L.fp8_amax_history_update_reset(self.hist[0:e], am[0:e], 0, 0, 0,
                                                            s[0:e], si[0:e])))
        ops.append(("delayed history E5M2", "state", 8.0 * 16 * (len(self.scale) - e),
                    lambda: L.fp8_amax_history_update_reset(self.hist[e:], am[e:], 1, 0, 0,
                                                            s[e:], si[e:])))
        return ops

    def _block_ops(self):
        L, T = self.L, self.T
        ops = []
        for n in C5_ORDER:
            di, do = self.shapes[n]
            xn = C5_X[n]
            if xn == n:
                ops.append((f"block cast X {n}", "cast", T * di * (4 + 8 / 128),
                            lambda xn=xn: L.fp8_cast_block(self.x[xn], 0, 1, self.xq[xn], self.sx[xn],
                                                           self.xtq[xn], self.sxt[xn])))
            ops.append((f"block cast W {n}", "cast", di * do * (4 + 8 / 16384),
                        lambda n=n: L.fp8_cast_block(self.w[n], 0, 2, self.wq[n], self.sw[n],
                                                     self.wtq[n], self.swt[n])))
            ops.append((f"block fwd {n}", "gemm", 2.0 * T * di * do,
                        lambda n=n, xn=xn: L.fp8_scaled_gemm(self.xq[xn], 0, 1, self.sx[xn],
                                                             self.wtq[n], 0, 2, self.swt[n], self.y[n])))
        for n in reversed(C5_ORDER):
            di, do = self.shapes[n]
            xn = C5_X[n]
            ops.append((f"block cast dY {n}", "cast", T * do * (4 + 8 / 128),
                        lambda n=n: L.fp8_cast_block(self.dy[n], 1, 1, self.dyq[n], self.sd[n],
                                                     self.dytq[n], self.sdt[n])))
            ops.append((f"block dgrad {n}", "gemm", 2.0 * T * di * do,
                        lambda n=n: L.fp8_scaled_gemm(self.dyq[n], 1, 1, self.sd[n], self.wq[n], 0, 2,
                                                      self.sw[n], self.dx[n])))
            ops.append((f"block wgrad {n}", "gemm", 2.0 * T * di * do,
                        lambda n=n, xn=xn: L.fp8_scaled_gemm(self.xtq[xn], 0, 1, self.sxt[xn],
                                                             self.dytq[n], 1, 1, self.sdt[n],
                                                             self.dw[n])))
        return ops

    def step(self):
        for mode in ("delayed", "block"):
            for _, _, _, fn in self.ops[mode]:
                fn()

    def timed_eager_step(self, stream):
        """One step with HIP events around every launch (on the library's
        stream); returns [(label, kind, work, seconds)]."""
        torch = self.torch
        evs = []
        # keep the GPU busy while the first launches are enqueued, so the
        # first event pair times the kernel, not the host's submission
        try:
            torch.cuda._sleep(4_000_000)
        except (AttributeError, RuntimeError):
            pass
        for mode in ("delayed", "block"):
            for lab, kind, work, fn in self.ops[mode]:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn()
                b.record(stream)
                evs.append((lab, kind, work, a, b))
        torch.cuda.synchronize()
        return [(lab, kind, work, a.elapsed_time(b) * 1e-3) for lab, kind, work, a, b in evs]


def c5_plan(T=8192):
    """The launches of one step in order, (label, kind, work), from the
    shapes alone (the op lists of C5Set follow it)."""
    from fp8_mixed_precision_linear_amd import datagen
    sh = datagen.C5_LINEARS
    plan = []
    for n in C5_ORDER:
        di, do = sh[n]
        if C5_X[n] == n:
            plan.append((f"delayed cast X {n}", "cast", 4.0 * T * di))
        plan.append((f"delayed cast W {n}", "cast", 4.0 * di * do))
        plan.append((f"delayed fwd {n}", "gemm", 2.0 * T * di * do))
    for n in reversed(C5_ORDER):
        di, do = sh[n]
        plan += [(f"delayed cast dY {n}", "cast", 4.0 * T * do),
                 (f"delayed dgrad {n}", "gemm", 2.0 * T * di * do),
                 (f"delayed wgrad {n}", "gemm", 2.0 * T * di * do)]
    n_e4m3 = len(set(C5_X.values())) + len(C5_ORDER)
    plan += [("delayed history E4M3", "state", 8.0 * 16 * n_e4m3),
             ("delayed history E5M2", "state", 8.0 * 16 * len(C5_ORDER))]
    for n in C5_ORDER:
        di, do = sh[n]
        if C5_X[n] == n:
            plan.append((f"block cast X {n}", "cast", T * di * (4 + 8 / 128)))
        plan.append((f"block cast W {n}", "cast", di * do * (4 + 8 / 16384)))
        plan.append((f"block fwd {n}", "gemm", 2.0 * T * di * do))
    for n in reversed(C5_ORDER):
        di, do = sh[n]
        plan += [(f"block cast dY {n}", "cast", T * do * (4 + 8 / 128)),
                 (f"block dgrad {n}", "gemm", 2.0 * T * di * do),
                 (f"block wgrad {n}", "gemm", 2.0 * T * di * do)]
    return plan


# GEMM kernel (instantiation) of each pass: the dominant-kernel roofline is
# taken over the launches of one kernel
C5_KERNEL = {
    "delayed fwd": "k_gemm_w4<0, 0, false, false, 0>",
    "delayed dgrad": "k_gemm_w4<1, 0, false, false, 0>",
    "delayed wgrad": "k_gemm_w4<0, 1, false, false, 0>",
    "block fwd": "k_gemm_big<0, 0, true, true, false, false, false>",
    "block dgrad": "k_gemm_big<1, 0, true, true, false, false, false>",
    "block wgrad": "k_gemm_big<0, 1, true, true, true, false, false>",
}


def c5_summary(timed):
    """Per-pass and per-kernel aggregates of one eager step's launches."""
    out = {"launches": {}}
    for lab, kind, work, sec in timed:
        e = {"us": round(sec * 1e6, 1)}
        if kind == "gemm":
            e["tflops"] = round(work / sec / 1e12, 1)
            e["pct_fp8_peak"] = round(100 * work / sec / 1e12 / FP8_PEAK_TFLOPS, 2)
        elif kind == "cast":
            e["gbs"] = round(work / sec / 1e9, 1)
            e["pct_hbm_peak"] = round(100 * work / sec / 1e9 / HBM_PEAK_GBS, 2)
        out["launches"][lab] = e
    for mode in ("delayed", "block"):
        g = [(w, s) for lab, k, w, s in timed if lab.startswith(mode) and k == "gemm"]
        c = [(w, s) for lab, k, w, s in timed if lab.startswith(mode) and k == "cast"]
        o = [s for lab, k, w, s in timed if lab.startswith(mode) and k == "state"]
        gw, gs = sum(w for w, _ in g), sum(s for _, s in g)
        cw, cs = sum(w for w, _ in c), sum(s for _, s in c)
        out[mode] = {"gemm_tflops": round(gw / gs / 1e12, 1), "gemm_ms": round(gs * 1e3, 3),
                     "gemm_pct_fp8_peak": round(100 * gw / gs / 1e12 / FP8_PEAK_TFLOPS, 2),
                     "cast_gbs": round(cw / cs / 1e9, 1), "cast_ms": round(cs * 1e3, 3),
                     "cast_pct_hbm_peak": round(100 * cw / cs / 1e9 / HBM_PEAK_GBS, 2),
                     "other_ms": round(sum(o) * 1e3, 3),
                     "sum_of_launches_ms": round((gs + cs + sum(o)) * 1e3, 3)}
    kern = {}
    for cls, name in C5_KERNEL.items():
        sel = [(w, s) for lab, k, w, s in timed if lab.startswith(cls + " ")]
        w, s = sum(x for x, _ in sel), sum(y for _, y in sel)
        kern[cls] = {"kernel": name, "launches": len(sel), "total_us": round(s * 1e6, 1),
                     "avg_us": round(s / len(sel) * 1e6, 1), "flop_per_launch": w / len(sel),
                     "tflops": round(w / s / 1e12, 1)}
    out["gemm_kernels"] = kern
    return out


def bench_c5(args, torch, L, datagen, dev, stream):
    c5 = C5Set(torch, L, datagen, dev)
    print(f"# generated the linear set's inputs in {c5.gen_s:.1f}s", file=sys.stderr, flush=True)
    for _ in range(max(1, args.warmup)):     # the first step fills the histories
        c5.step()
    torch.cuda.synchronize()
    g = capture(torch, lambda: [c5.step() for _ in range(args.steps)])
    g.replay()                               # first replay uploads the graph
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    ev0.record(stream)
    g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    print(f"# C5 step {ms_step:.3f} ms (graph)", file=sys.stderr, flush=True)
    clock = sample_clock_under(torch, g)
    del g
    timed = c5.timed_eager_step(stream)
    summ = c5_summary(timed)
    flops = 2 * c5.flops_per_pass()
    cast_bytes = sum(w for mode in ("delayed", "block") for _, k, w, _ in c5.ops[mode] if k == "cast")
    dom_cls = max(summ["gemm_kernels"], key=lambda k: summ["gemm_kernels"][k]["total_us"])
    dom = summ["gemm_kernels"][dom_cls]
    ach = dom["flop_per_launch"] / (dom["avg_us"] * 1e-6) / 1e12
    roofline = {"bound": "mfma", "kernel": f"{dom['kernel']} ({dom_cls}, 5 launches per step)",
                "achieved": round(ach, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / FP8_PEAK_TFLOPS, 4),
                "traffic": gemm_traffic(dom_cls)}
    del c5
    torch.cuda.empty_cache()
    return {"ms_step": ms_step, "flops": flops, "cast_bytes": cast_bytes, "wall": wall,
            "summary": summ, "roofline": roofline, "clock": clock}


# ----------------------------------------------------------------------------
# extras: the 4096^3 delayed-scaling step, per-kernel timings, row-wise and
# block-wise paths at the smaller sizes
# ----------------------------------------------------------------------------
def bench_extras(args, torch, L, datagen, dev, stream):
    def d_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    T = DI = DO = 4096
    NSTEPS_DATA = 16
    t0 = time.time()
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        steps = list(ex.map(datagen.config2_step, range(NSTEPS_DATA)))
    data = [(d_bf16(s["x"]), d_bf16(s["w"]), d_bf16(s["dy"])) for s in steps]
    del steps
    print(f"# generated 16 steps of 4096^3 inputs in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)
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

    for t in range(4):
        step(t)
    torch.cuda.synchronize()
    nst = 32
    g = capture(torch, lambda: [step(4 + t) for t in range(nst)])
    g.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / nst
    del g
    delayed4096 = {"workload": "delayed-scaling fwd+dgrad+wgrad, tokens 4096, in 4096, out 4096, "
                               "16 steps of inputs regenerated per step (graph of 32 steps)",
                   "ms_per_step": round(ms_step, 4),
                   "tflops_incl_casts": round(3 * 2.0 * T * DI * DO / (ms_step * 1e-3) / 1e12, 2)}

    def time_launch(fn, reps, replays=3):
        g = capture(torch, lambda: [fn() for _ in range(reps)])
        g.replay()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(replays):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(b))
        del g
        return best / reps * 1e-3

    x0, w0, dy0 = data[0]
    R = args.kernel_reps
    k = {}
    k["gemm_fwd_tensor"] = time_launch(lambda: L.fp8_scaled_gemm(xq, 0, 0, sinv[0:1], wtq, 0, 0, sinv[1:2], y), R)
    k["gemm_dgrad_tensor"] = time_launch(lambda: L.fp8_scaled_gemm(dyq, 1, 0, sinv[2:3], wq, 0, 0, sinv[1:2], dx), R)
    k["gemm_wgrad_tensor"] = time_launch(lambda: L.fp8_scaled_gemm(xtq, 0, 0, sinv[0:1], dytq, 1, 0, sinv[2:3], dw), R)
    y8, y8t = torch.empty((T, DO), **u8), torch.empty((DO, T), **u8)
    am8 = torch.zeros(1, dtype=torch.float32, device=dev)
    # the quantising epilogue (E4M3 codes, transposed copy, amax
    # max-accumulated into the slot as in a delayed-scaling step), timed
    # right after the same GEMM with a BF16 output; then with the amax
    # overwritten (a one-word fill launched ahead of the GEMM)
    fp8out = (lambda: L.fp8_scaled_gemm(xq, 0, 0, sinv[0:1], wtq, 0, 0, sinv[1:2], y8, d_amax=am8,
                                        d_scale=scale[0:1], d_fmt=0, D_t=y8t, amax_accumulate=True))
    k["gemm_fwd_tensor_fp8out"] = float("inf")
    for _ in range(2):   # interleaved with the BF16-output GEMM, best of each
        k["gemm_fwd_tensor"] = min(k["gemm_fwd_tensor"], time_launch(
            lambda: L.fp8_scaled_gemm(xq, 0, 0, sinv[0:1], wtq, 0, 0, sinv[1:2], y), R))
        k["gemm_fwd_tensor_fp8out"] = min(k["gemm_fwd_tensor_fp8out"], time_launch(fp8out, R))
    k["gemm_fwd_tensor_fp8out_amax_overwrite"] = time_launch(
        lambda: L.fp8_scaled_gemm(xq, 0, 0, sinv[0:1], wtq, 0, 0, sinv[1:2], y8, d_amax=am8,
                                  d_scale=scale[0:1], d_fmt=0, D_t=y8t), R)
    k["cast_transpose_amax_e4m3"] = time_launch(lambda: L.fp8_cast_e4m3(x0, scale[0:1], y=xq, y_t=xtq, amax_out=amax[0:1]), R)
    k["cast_transpose_amax_acc_e4m3"] = time_launch(lambda: L.fp8_cast_amax_acc(x0, 0, scale[0:1], amax[0:1], y=xq, y_t=xtq), R)
    k["cast_transpose_amax_e5m2_sr"] = time_launch(
        lambda: L.fp8_cast_sr(dy0, 1, scale[2:3], 1234, 0, y=dyq, y_t=dytq, amax_out=amax[2:3]), R)
    k["cast_e4m3"] = time_launch(lambda: L.fp8_cast_e4m3(x0, scale[0:1], y=xq), R)
    k["amax"] = time_launch(lambda: L.fp8_amax_acc(x0, amax[0:1]), R)
    k["amax_overwrite"] = time_launch(lambda: L.fp8_amax(x0, amax[0:1]), R)
    k["history_update"] = time_launch(lambda: L.fp8_amax_history_update(hist[0:2], amax[0:2], 0, 0, 0, scale[0:2], sinv[0:2]), R)
    ewma = torch.zeros(3, dtype=torch.float32, device=dev)
    k["ewma_update"] = time_launch(lambda: L.fp8_amax_ewma_update(ewma, amax, 0.9, 0, 0, scale, sinv), R)
    nel = T * DI
    fl = 2.0 * T * DI * DO
    kernels = {"note": "warm: R launches back to back in one HIP graph, best of 3 replays"}
    for n in ("gemm_fwd_tensor", "gemm_dgrad_tensor", "gemm_wgrad_tensor", "gemm_fwd_tensor_fp8out",
              "gemm_fwd_tensor_fp8out_amax_overwrite"):
        kernels[n] = {"tflops": round(fl / k[n] / 1e12, 2), "us": round(k[n] * 1e6, 2)}
    kernels["gemm_fwd_tensor_fp8out"]["us_unfused_equivalent"] = round(
        (k["gemm_fwd_tensor"] + k["cast_transpose_amax_acc_e4m3"]) * 1e6, 2)
    kernels["gemm_fwd_tensor_fp8out"]["vs_bf16_out"] = round(k["gemm_fwd_tensor_fp8out"] / k["gemm_fwd_tensor"], 3)
    for n, bpe in (("cast_transpose_amax_e4m3", 4), ("cast_transpose_amax_acc_e4m3", 4),
                   ("cast_transpose_amax_e5m2_sr", 4), ("cast_e4m3", 3), ("amax", 2),
                   ("amax_overwrite", 2)):
        kernels[n] = {"gbs": round(bpe * nel / k[n] / 1e9, 1), "us": round(k[n] * 1e6, 2)}
    kernels["history_update"] = {"us": round(k["history_update"] * 1e6, 2)}
    kernels["ewma_update"] = {"us": round(k["ewma_update"] * 1e6, 2)}

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
    rowwise = rowwise_summary(k, T, DI, DO, "row-wise fwd+dgrad+wgrad, tokens 4096, in 4096, out 4096")

    # cold: a 512 MiB read evicts the 256 MB MALL with clean lines before
    # every timed launch; each launch bracketed by its own HIP events
    flush = torch.zeros(256 << 20, dtype=torch.bfloat16, device=dev)
    flush_amax = torch.zeros(1, dtype=torch.float32, device=dev)

    def time_cold(fn, reps):
        evs = []
        for _ in range(reps):
            L.fp8_amax(flush, flush_amax)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in evs)
        return ts[len(ts) // 2] * 1e-3

    kc = {}
    kc["gemm_fwd_tensor"] = time_cold(lambda: L.fp8_scaled_gemm(xq, 0, 0, sinv[0:1], wtq, 0, 0, sinv[1:2], y), R)
    kc["gemm_dgrad_tensor"] = time_cold(lambda: L.fp8_scaled_gemm(dyq, 1, 0, sinv[2:3], wq, 0, 0, sinv[1:2], dx), R)
    kc["gemm_wgrad_tensor"] = time_cold(lambda: L.fp8_scaled_gemm(xtq, 0, 0, sinv[0:1], dytq, 1, 0, sinv[2:3], dw), R)
    kc["cast_transpose_amax_acc_e4m3"] = time_cold(lambda: L.fp8_cast_amax_acc(x0, 0, scale[0:1], amax[0:1], y=xq, y_t=xtq), R)
    kc["cast_e4m3"] = time_cold(lambda: L.fp8_cast_e4m3(x0, scale[0:1], y=xq), R)
    kc["amax"] = time_cold(lambda: L.fp8_amax_acc(x0, amax[0:1]), R)
    kc["cast_rowwise_dy"] = time_cold(lambda: L.fp8_cast_rowwise(dy0, 1, dyq, sdr, dytq, sdc), R)
    # the same bytes as the cast-transpose (2 B/elem read, 2 written) through
    # a plain device copy: the practical ceiling of that traffic pattern
    x0c = torch.empty_like(x0)
    kc["copy_same_bytes"] = time_cold(lambda: x0c.copy_(x0), R)
    kernels_cold = {"note": "MALL evicted (512 MiB read) before every timed launch; median of "
                            f"{R} single launches, each bracketed by HIP events"}
    for n in ("gemm_fwd_tensor", "gemm_dgrad_tensor", "gemm_wgrad_tensor"):
        kernels_cold[n] = {"tflops": round(fl / kc[n] / 1e12, 2), "us": round(kc[n] * 1e6, 2)}
    for n, by in (("cast_transpose_amax_acc_e4m3", 4.0 * nel), ("cast_e4m3", 3.0 * nel),
                  ("amax", 2.0 * nel), ("cast_rowwise_dy", 4.0 * nel + 4.0 * (T + DO)),
                  ("copy_same_bytes", 4.0 * nel)):
        kernels_cold[n] = {"gbs": round(by / kc[n] / 1e9, 1), "us": round(kc[n] * 1e6, 2),
                           "pct_hbm_peak": round(100 * by / kc[n] / 1e9 / HBM_PEAK_GBS, 2)}
    kernels_cold["cast_transpose_amax_acc_e4m3"]["vs_copy_same_bytes"] = round(
        kc["copy_same_bytes"] / kc["cast_transpose_amax_acc_e4m3"], 3)
    del x0c
    del data
    blockwise = bench_blockwise(torch, L, datagen, dev, d_bf16, time_launch, time_cold, R)
    del flush
    c1 = bench_config1(torch, L, datagen, dev, d_bf16, stream)
    return {"config1": c1, "delayed4096": delayed4096, "kernels": kernels, "kernels_cold": kernels_cold,
            "rowwise": rowwise, "blockwise": blockwise}


def bench_config1(torch, L, datagen, dev, d_bf16, stream):
    """Latency of the per-tensor current-scaling forward at X 256x512,
    W 512x512: amax of X and W (max-accumulated into a zeroed pair), both
    scales in one call, the cast of X, the transposed cast of W, the GEMM
    with BF16 output -- 7 kernels, timed as a replayed HIP graph and as
    eager calls through the binding."""
    c = datagen.config1()
    x, w = d_bf16(c["x"]), d_bf16(c["w"])
    u8 = dict(dtype=torch.uint8, device=dev)
    amax = torch.zeros(2, dtype=torch.float32, device=dev)
    s, si = torch.ones(2, dtype=torch.float32, device=dev), torch.ones(2, dtype=torch.float32, device=dev)
    xq, wtq = torch.empty((256, 512), **u8), torch.empty((512, 512), **u8)
    y = torch.empty((256, 512), dtype=torch.bfloat16, device=dev)

    def fwd():
        amax.zero_()
        L.fp8_amax_acc(x, amax[0:1])
        L.fp8_amax_acc(w, amax[1:2])
        L.fp8_compute_scale(amax, 0, 0, s, si)
        L.fp8_cast_e4m3(x, s[0:1], y=xq)
        L.fp8_cast_e4m3(w, s[1:2], y_t=wtq)
        L.fp8_scaled_gemm(xq, 0, 0, si[0:1], wtq, 0, 0, si[1:2], y)

    n = 100
    g = capture(torch, lambda: [fwd() for _ in range(n)])
    g.replay()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b) / n)
    del g
    for _ in range(5):
        fwd()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        fwd()
    torch.cuda.synchronize()
    eager = (time.perf_counter() - t0) / n
    return {"workload": "per-tensor current-scaling forward, X 256x512 (4 outlier columns x50), "
                        "W 512x512: amax x2, scales, cast, cast-transpose, GEMM (7 kernels)",
            "us_per_forward_graph": round(best * 1e3, 2),
            "us_per_forward_eager": round(eager * 1e6, 2),
            "gflop": round(2.0 * 256 * 512 * 512 / 1e9, 3)}


def bench_blockwise(torch, L, datagen, dev, d_bf16, time_launch, time_cold, R):
    T, DI, DO = 8192, 4096, 14336
    c3 = datagen.config3()
    x, w = d_bf16(c3["x"]), d_bf16(c3["w"])
    dy = d_bf16(datagen.config4_dy(c3["rng"]))
    del c3
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
    k, kc = {}, {}
    casts = {
        "cast_block_x_dual": (lambda: L.fp8_cast_block(x, 0, 1, xq, sx, xtq, sxt), T * DI * (4 + 8 / 128)),
        "cast_block_w_128x128_both": (lambda: L.fp8_cast_block(w, 0, 2, wq, sw, wtq, swt), DI * DO * (4 + 8 / 16384)),
        "cast_block_dy_dual": (lambda: L.fp8_cast_block(dy, 1, 1, dyq, sdy, dytq, sdyt), T * DO * (4 + 8 / 128)),
        "cast_block_pow2_dy_dual": (lambda: L.fp8_cast_block_pow2(dy, 1, 1, dyq, sdy, dytq, sdyt), T * DO * (4 + 8 / 128)),
        "cast_rowwise_dy": (lambda: L.fp8_cast_rowwise(dy, 1, dyq, sdy[0], dytq, sdyt[0]), T * DO * 4.0 + 4.0 * (T + DO)),
    }
    for n, (fn, _) in casts.items():
        k[n] = time_launch(fn, R)
        kc[n] = time_cold(fn, R)
    L.fp8_cast_block(x, 0, 1, xq, sx, xtq, sxt)
    L.fp8_cast_block(w, 0, 2, wq, sw, wtq, swt)
    L.fp8_cast_block(dy, 1, 1, dyq, sdy, dytq, sdyt)
    gem = {
        "gemm_fwd_block": lambda: L.fp8_scaled_gemm(xq, 0, 1, sx, wtq, 0, 2, swt, y),
        "gemm_dgrad_block": lambda: L.fp8_scaled_gemm(dyq, 1, 1, sdy, wq, 0, 2, sw, dx),
        "gemm_wgrad_block": lambda: L.fp8_scaled_gemm(xtq, 0, 1, sxt, dytq, 1, 1, sdyt, dw),
    }
    for n, fn in gem.items():
        k[n] = time_launch(fn, R)
    L.fp8_cast_block_pow2(x, 0, 1, xq, sx, xtq, sxt)
    L.fp8_cast_block_pow2(w, 0, 2, wq, sw, wtq, swt)
    L.fp8_cast_block_pow2(dy, 1, 1, dyq, sdy, dytq, sdyt)
    gem2 = {
        "gemm_fwd_block_pow2": lambda: L.fp8_scaled_gemm(xq, 0, 3, sx, wtq, 0, 4, swt, y),
        "gemm_dgrad_block_pow2": lambda: L.fp8_scaled_gemm(dyq, 1, 3, sdy, wq, 0, 4, sw, dx),
        "gemm_wgrad_block_pow2": lambda: L.fp8_scaled_gemm(xtq, 0, 3, sxt, dytq, 1, 3, sdyt, dw),
    }
    for n, fn in gem2.items():
        k[n] = time_launch(fn, R)
    fl = 2.0 * T * DI * DO
    out = {"workload": "block-wise fwd (X 8192x4096 Student-t 1x128, W 4096x14336 128x128) + "
                       "bwd (dY 8192x14336 1x128 dual orientation; dgrad, wgrad)"}
    for n in list(gem) + list(gem2):
        out[n] = {"tflops": round(fl / k[n] / 1e12, 2), "us": round(k[n] * 1e6, 1),
                  "pct_fp8_peak": round(100 * fl / k[n] / 1e12 / FP8_PEAK_TFLOPS, 2)}
    for n, (_, by) in casts.items():
        out[n] = {"gbs_cold": round(by / kc[n] / 1e9, 1), "us_cold": round(kc[n] * 1e6, 1),
                  "pct_hbm_peak_cold": round(100 * by / kc[n] / 1e9 / HBM_PEAK_GBS, 2),
                  "gbs_warm": round(by / k[n] / 1e9, 1), "us_warm": round(k[n] * 1e6, 1)}
    return out


def rowwise_summary(k, T, DI, DO, workload):
    fl = 2.0 * T * DI * DO
    out = {"workload": workload}
    for n in ("gemm_fwd_rowwise", "gemm_dgrad_rowwise", "gemm_wgrad_rowwise"):
        out[n] = {"tflops": round(fl / k[n] / 1e12, 2), "us": round(k[n] * 1e6, 1)}
    shapes = {"cast_rowwise_x": (T, DI), "cast_rowwise_w": (DI, DO), "cast_rowwise_dy": (T, DO)}
    for n, (a, b) in shapes.items():
        by = a * b * 4.0 + 4.0 * (a + b)
        out[n] = {"gbs": round(by / k[n] / 1e9, 1), "us": round(k[n] * 1e6, 1)}
    return out


# ----------------------------------------------------------------------------
# HBM traffic of the step's GEMM kernels (rocprofv3 counter runs)
# ----------------------------------------------------------------------------
def traffic_sources_sha256() -> str:
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "fp8_mixed_precision_linear_amd", rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def gemm_traffic(cls):
    """Measured HBM bytes per launch of a GEMM kernel of the step (average
    over its five launches), from the committed counter summary, or None
    when the kernel sources changed after the counters were taken."""
    try:
        with open(TRAFFIC_JSON) as f:
            t = json.load(f)
        if t.get("sources_sha256") != traffic_sources_sha256():
            return None
        k = t["kernels"][cls]
        return round(k["traffic_bytes"] / k["launches"])
    except (OSError, KeyError, ValueError):
        return None


COPY_BYTES = 256 << 20


def traffic_run():
    """Under rocprofv3 --pmc: a copy of known size (256 MiB read, 256 MiB
    written); then per pass the step's casts and history updates once and
    each GEMM twice (the summary keeps the second launch); then the
    row-wise cast of the O linear's activation (8192 x 8192, both
    orientations) twice."""
    import torch
    from fp8_mixed_precision_linear_amd import datagen
    from fp8_mixed_precision_linear_amd import lib as L
    dev = torch.device("cuda:0")
    xin = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    xout = torch.empty_like(xin)
    for _ in range(3):
        torch.neg(xin, out=xout)
    torch.cuda.synchronize()
    del xin, xout
    c5 = C5Set(torch, L, datagen, dev)
    for mode in ("delayed", "block"):
        for lab, kind, work, fn in c5.ops[mode]:
            if kind != "gemm":
                fn()
        for lab, kind, work, fn in c5.ops[mode]:
            if kind == "gemm":
                fn()
                fn()
        torch.cuda.synchronize()
    x = c5.x["o"]
    T, DI = x.shape
    f32 = dict(dtype=torch.float32, device=dev)
    sr, sc = torch.empty(T, **f32), torch.empty(DI, **f32)
    for _ in range(2):
        L.fp8_cast_rowwise(x, 0, c5.xq["o"], sr, c5.xtq["o"], sc)
    torch.cuda.synchronize()
    print("traffic-run: done", flush=True)


def traffic_summarize(d, dst):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE of traffic_run's program ->
    bytes per launch of each GEMM kernel of the step (average over its five
    linears), of each cast kind, and of the row-wise cast's kernels."""
    import re

    def per_dispatch(sub, counter):
        files = glob.glob(os.path.join(d, sub, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise FileNotFoundError(f"no counter_collection.csv under {os.path.join(d, sub)}")
        vals = {}
        for f in files:
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                vals.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], 0.0])
                vals[int(r["Dispatch_Id"])][1] += float(r["Counter_Value"])
        return [vals[i] for i in sorted(vals)]

    def nospace(t):
        return re.sub(r"\s", "", t)

    def classify(rows):
        """(copy values, {class: [values]}): the launches in traffic_run's
        order, each checked against the kernel it must be."""
        copy = [v for n, v in rows if "neg_kernel" in n]
        ours = [(n, v) for n, v in rows if "fp8lin" in n]
        plan = c5_plan()
        seq = []
        for mode in ("delayed", "block"):
            seq += [(lab, k, w) for lab, k, w in plan if lab.startswith(mode) and k != "gemm"]
            for lab, k, w in plan:
                if lab.startswith(mode) and k == "gemm":
                    seq += [(lab + " (first)", k, w), (lab, k, w)]
        rw = ["k_rw_rows", "k_rw_colmax", "k_rw_transpose", "k_rw_finalize"]
        seq += [(f"rowwise {k}", "rowwise", 0.0) for _ in range(2) for k in rw]
        assert len(ours) == len(seq), (len(ours), len(seq))
        out = {}
        for (name, v), (lab, kind, w) in zip(ours, seq):
            if lab.endswith("(first)"):
                continue
            if kind == "gemm":
                cls = lab.rsplit(" ", 1)[0]
                assert nospace(C5_KERNEL[cls]) in nospace(name), (lab, name)
            elif kind == "cast":
                cls = lab.rsplit(" ", 1)[0]
                want = "k_cast_transpose" if cls.startswith("delayed") else (
                    "k_cast_block<0,2" if cls.endswith("W") else "k_cast_block<")
                assert want in nospace(name), (lab, name)
            elif kind == "state":
                cls = "delayed history"
                assert "k_history_update" in name, (lab, name)
            else:
                cls = lab
                assert lab.split(" ")[1] in name, (lab, name)
            out.setdefault(cls, []).append((v, w))
        return (copy[1:] if len(copy) > 1 else copy), out

    fcopy, fetch = classify(per_dispatch("fetch", "FETCH_SIZE"))
    wcopy, write = classify(per_dispatch("write", "WRITE_SIZE"))
    kib = COPY_BYTES / 1024.0
    f_fetch = kib / (sum(fcopy) / len(fcopy))
    f_write = kib / (sum(wcopy) / len(wcopy))
    from fp8_mixed_precision_linear_amd import datagen
    T = 8192

    def gemm_alg(cls):
        alg = 0.0
        for n in C5_ORDER:
            di, do = datagen.C5_LINEARS[n]
            if cls.endswith("fwd"):
                alg += T * di + do * di + 2 * T * do
            elif cls.endswith("dgrad"):
                alg += T * do + di * do + 2 * T * di
            else:
                alg += di * T + do * T + 4 * di * do
        return alg / 5

    res = {"what": "HBM bytes per launch (FETCH_SIZE and WRITE_SIZE, KiB per dispatch, each scaled "
                   "by the reading for a 256 MiB elementwise copy (neg) of known size): the GEMM "
                   "kernels of the transformer-block step (average over its five linears), its "
                   "casts per kind, and the row-wise cast of an 8192 x 8192 activation",
           "copy_scale": {"fetch": round(f_fetch, 4), "write": round(f_write, 4)},
           "sources_sha256": traffic_sources_sha256(), "kernels": {}, "casts": {}, "rowwise": {}}
    for cls in fetch:
        nf = len(fetch[cls])
        rd = sum(v for v, _ in fetch[cls]) / nf * f_fetch * 1024.0
        wr = sum(v for v, _ in write[cls]) / nf * f_write * 1024.0
        if cls in C5_KERNEL:
            alg = gemm_alg(cls)
            key = "kernels"
            extra = {"kernel": C5_KERNEL[cls]}
        elif cls.startswith("rowwise"):
            alg = None
            key = "rowwise"
            extra = {}
        elif cls == "delayed history":
            continue
        else:
            alg = sum(w for _, w in fetch[cls]) / nf
            key = "casts"
            extra = {}
        e = {**extra, "launches": nf, "read_bytes": round(rd), "write_bytes": round(wr),
             "traffic_bytes": round(rd + wr)}
        if alg:
            e["algorithmic_bytes"] = round(alg)
            e["traffic_over_algorithmic"] = round((rd + wr) / alg, 3)
        res[key][cls] = e
    rw = res["rowwise"]
    if rw:
        tot = sum(e["traffic_bytes"] for e in rw.values())
        alg = 8192 * 8192 * 4.0 + 4.0 * 2 * 8192
        rw["total"] = {"traffic_bytes": tot, "algorithmic_bytes": round(alg),
                       "traffic_over_algorithmic": round(tot / alg, 3)}
    with open(dst, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


# ----------------------------------------------------------------------------
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


def amd_smi_gfx_mhz():
    """Current gfx clock of GPU 0, MHz, averaged over its XCDs, from the
    amd-smi tool (a child process); None when it is not available."""
    try:
        out = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--json"],
                             capture_output=True, text=True, timeout=20).stdout
        clk = json.loads(out)["gpu_data"][0]["clock"]
        vals = [v["clk"]["value"] for k, v in clk.items() if k.startswith("gfx_")]
        vals = [float(v) for v in vals if isinstance(v, (int, float))]
        return sum(vals) / len(vals) if vals else None
    except Exception:
        return None


def sample_clock_under(torch, g, max_replays=40):
    """The gfx clock while the step runs: the captured step is replayed back
    to back while a thread samples amd-smi twice; replays continue until the
    samples are in (at most max_replays)."""
    import threading
    samples = []

    def sampler():
        for _ in range(2):
            time.sleep(0.3)
            v = amd_smi_gfx_mhz()
            if v is not None:
                samples.append(v)

    th = threading.Thread(target=sampler)
    th.start()
    n = 0
    while th.is_alive() and n < max_replays:
        g.replay()
        torch.cuda.synchronize()
        n += 1
    th.join()
    return {"gfx_mhz_under_load": round(sum(samples) / len(samples), 1) if samples else None,
            "samples": len(samples), "source": "amd-smi metric --clock (mean over the 8 XCDs)",
            "step_replays_during_sampling": n}


def cpu_model() -> str:
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    return "unknown"


def cpu_baseline(step_flops, step_cast_bytes):
    """The oracle, as it stands, on a bounded sample of the step: the O
    linear (8192 tokens, 8192 -> 8192) in both passes -- the casts of X, W
    and dY at full size (per-tensor with transpose, and block-wise) and the
    three GEMMs of each pass on 192 of 8192 output rows -- extrapolated to
    the step: GEMM time by FLOPs, cast time by algorithmic bytes."""
    from fp8_mixed_precision_linear_amd import datagen
    from oracle import oracle as O
    d = datagen.config5_linear("o")
    x, w, dy = d["x"], d["w"], d["dy"]
    T, DI = x.shape
    DO = w.shape[1]
    t0 = time.perf_counter()
    ax, aw, ad = O.amax_parallel(x), O.amax_parallel(w), O.amax_parallel(dy)
    sx, sxi, _ = O.compute_scale(ax, 0)
    sw, swi, _ = O.compute_scale(aw, 0)
    sd, sdi, _ = O.compute_scale(ad, 1)
    xq, wq, dq = O.cast(x, sx, 0), O.cast(w, sw, 0), O.cast(dy, sd, 1)
    bx = O.cast_block(x, 0, O.S1x128, want_y=True, want_t=True)
    bw = O.cast_block(w, 0, O.S128x128, want_y=True, want_t=True)
    bd = O.cast_block(dy, 1, O.S1x128, want_y=True, want_t=True)
    t_cast = time.perf_counter() - t0
    cast_bytes = 2 * 4.0 * (T * DI + DI * DO + T * DO)   # both passes, both orientations
    rows = np.arange(192, dtype=np.int64)
    t1 = time.perf_counter()
    one = lambda v: np.array([v], np.float32)
    xt, dt_, wt = (np.ascontiguousarray(a.T) for a in (xq, dq, wq))
    O.gemm(xq, 0, 0, one(sxi), wt, 0, 0, one(swi), ms=rows)
    O.gemm(dq, 1, 0, one(sdi), wq, 0, 0, one(swi), ms=rows)
    O.gemm(xt, 0, 0, one(sxi), dt_, 1, 0, one(sdi), ms=rows)
    O.gemm(bx["y"], 0, 1, bx["sinv"], bw["y_t"], 0, 2, bw["sinv_t"], ms=rows)
    O.gemm(bd["y"], 1, 1, bd["sinv"], bw["y"], 0, 2, bw["sinv"], ms=rows)
    O.gemm(bx["y_t"], 0, 1, bx["sinv_t"], bd["y_t"], 1, 1, bd["sinv_t"], ms=rows)
    t_gemm_sample = time.perf_counter() - t1
    sample_flops = 6 * 2.0 * len(rows) * DO * DI   # each GEMM: 192 rows x 8192 x 8192
    t_step = t_gemm_sample * step_flops / sample_flops + t_cast * step_cast_bytes / cast_bytes
    return {"value": round(step_flops / t_step / 1e12, 6), "unit": "TFLOP/s", "cores": O.nthreads(),
            "kind": "oracle", "host_cpus": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": "the O linear (8192 tokens, 8192 -> 8192) in both passes: amax, scales and "
                      f"casts of X, W, dY at full size ({t_cast:.2f}s), the six GEMMs on {len(rows)} of "
                      f"8192 output rows ({t_gemm_sample:.2f}s); extrapolated to the step by FLOPs "
                      "(GEMMs) and algorithmic bytes (casts)",
            "step_s_extrapolated": round(t_step, 1)}


def main():
    args = parse()
    if args.traffic_summarize:
        traffic_summarize(*args.traffic_summarize)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the FP8 linear path here has no multi-GPU "
              "(sharded) mode; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.traffic_run:
        traffic_run()
        return

    import torch
    from fp8_mixed_precision_linear_amd import datagen
    from fp8_mixed_precision_linear_amd import lib as L

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    h = bench_c5(args, torch, L, datagen, dev, stream)
    value = h["flops"] / (h["ms_step"] * 1e-3) / 1e12
    summ = h["summary"]
    result = {
        "metric": "FP8 scaled-GEMM TFLOP/s (fwd+dgrad+wgrad, % FP8 peak) + cast GB/s",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(h["ms_step"], 4), "higher_is_better": True,
        "launch": "hip_graph", "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8-e4m3/e5m2 (fp32 accumulate)",
        "data": "synthetic (seeded numpy PCG64, bf16)",
        "config": {"workload": "transformer-block FP8 linear set, hidden 8192, FFN 28672, 8192 "
                               "tokens: QKV 8192->10240, O 8192->8192, gate/up 8192->28672 "
                               "(shared input), down 28672->8192; fwd+dgrad+wgrad of every "
                               "linear in per-tensor delayed scaling (history 16) and in "
                               "block-wise scaling (1x128 / 128x128); 2 x 42.06 TFLOP per step",
                   "global_batch": 8192, "seq_len": None, "parallelism": "none (1 GPU)"},
        "wall_s_timed": round(h["wall"], 4),
        "pct_fp8_peak": round(100 * value / FP8_PEAK_TFLOPS, 2),
        "roofline": h["roofline"],
        "clock": h["clock"],
        "c5": summ,
    }
    mhz = h["clock"].get("gfx_mhz_under_load")
    if mhz:   # the peaks assume 2.4 GHz; the same fractions at the clock the step ran at
        result["clock"]["pct_fp8_peak_at_measured_clock"] = round(
            100 * value / (FP8_PEAK_TFLOPS * mhz / 2400.0), 2)
        result["clock"]["roofline_frac_at_measured_clock"] = round(
            h["roofline"]["frac"] * 2400.0 / mhz, 4)
    if not args.no_extras:
        result.update(bench_extras(args, torch, L, datagen, dev, stream))
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(h["flops"], h["cast_bytes"])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
