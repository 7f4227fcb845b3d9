"""HBM traffic of the per-tensor FP8 GEMMs at 4096^3 and of the per-tensor
cast+transpose+amax at 4096 x 4096, from rocprofv3 counter runs.

Two counter passes over the same workload (FETCH_SIZE, then WRITE_SIZE: the
kilobytes the L2 reads from / writes to device memory per dispatch), then a
summary.  Each counter is scaled by what it reads for a plain elementwise
kernel of known size (out = -in over 256 MiB of bf16: 256 MiB read, 256 MiB
written), so the reported bytes are in the units of the algorithmic bytes.

  cd /tmp && export TMPDIR=/tmp && cd <repo>
  rocprofv3 --pmc FETCH_SIZE -f csv -d <dir>/fetch -o p -- \\
      python3 -m fp8_mixed_precision_linear_amd.traffic_probe run
  rocprofv3 --pmc WRITE_SIZE -f csv -d <dir>/write -o p -- \\
      python3 -m fp8_mixed_precision_linear_amd.traffic_probe run
  python3 -m fp8_mixed_precision_linear_amd.traffic_probe summarize <dir> \\
      profiles/gemm_tensor4096_traffic.json

The summary stores the SHA-256 of the kernel sources it measured; bench.py
reports the traffic only while those sources are unchanged.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 256 << 20
REPS = 3
SOURCES = ("csrc/gemm_big_kernel.h", "csrc/gemm_big.hip", "csrc/cast_kernels.hip",
           "csrc/fp8_device.h")


def sources_sha256() -> str:
    h = hashlib.sha256()
    for rel in SOURCES:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def run():
    import numpy as np
    import torch
    from fp8_mixed_precision_linear_amd import datagen
    from fp8_mixed_precision_linear_amd import lib as L

    dev = torch.device("cuda:0")
    xin = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    xout = torch.empty_like(xin)
    for _ in range(REPS):
        torch.neg(xin, out=xout)
    torch.cuda.synchronize()
    del xin, xout

    s = datagen.config2_step(0)
    def d_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    x, w, dy = d_bf16(s["x"]), d_bf16(s["w"]), d_bf16(s["dy"])
    T = 4096
    u8 = dict(dtype=torch.uint8, device=dev)
    xq, xtq, wq, wtq = (torch.empty((T, T), **u8) for _ in range(4))
    dyq, dytq = torch.empty((T, T), **u8), torch.empty((T, T), **u8)
    y = torch.empty((T, T), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((T, T), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((T, T), dtype=torch.float32, device=dev)
    sc = torch.ones(3, device=dev)
    am = torch.zeros(3, device=dev)
    for _ in range(REPS):
        L.fp8_cast_e4m3(x, sc[0:1], y=xq, y_t=xtq, amax_out=am[0:1])
        L.fp8_cast_e4m3(w, sc[1:2], y=wq, y_t=wtq, amax_out=am[1:2])
        L.fp8_cast_e5m2(dy, sc[2:3], y=dyq, y_t=dytq, amax_out=am[2:3])
    for _ in range(REPS):
        L.fp8_scaled_gemm(xq, 0, 0, sc[0:1], wtq, 0, 0, sc[1:2], y)
        L.fp8_scaled_gemm(dyq, 1, 0, sc[2:3], wq, 0, 0, sc[1:2], dx)
        L.fp8_scaled_gemm(xtq, 0, 0, sc[0:1], dytq, 1, 0, sc[2:3], dw)
    torch.cuda.synchronize()
    print("traffic_probe: done", flush=True)


def _classify(name: str):
    if "neg" in name and "elementwise" in name:
        return "copy"
    if "k_gemm_big<0, 0, false" in name:
        return "gemm_fwd_tensor"
    if "k_gemm_big<1, 0, false" in name:
        return "gemm_dgrad_tensor"
    if "k_gemm_big<0, 1, false" in name:
        return "gemm_wgrad_tensor"
    if "k_cast_transpose<0, true, true, false>" in name:
        return "cast_transpose_amax_e4m3"
    if "k_cast_transpose<1, true, true, false>" in name:
        return "cast_transpose_amax_e5m2"
    return None


def _per_dispatch(d: str, counter: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    vals = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            k = _classify(r["Kernel_Name"])
            if k is None:
                continue
            vals.setdefault(k, {}).setdefault(int(r["Dispatch_Id"]), 0.0)
            vals[k][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    # drop the first dispatch of each kernel (cold caches), average the rest
    out = {}
    for k, dd in vals.items():
        v = [dd[i] for i in sorted(dd)]
        v = v[1:] if len(v) > 1 else v
        out[k] = sum(v) / len(v)
    return out


def summarize(d: str, dst: str):
    fetch = _per_dispatch(os.path.join(d, "fetch"), "FETCH_SIZE")
    write = _per_dispatch(os.path.join(d, "write"), "WRITE_SIZE")
    kib = COPY_BYTES / 1024.0
    f_fetch = kib / fetch["copy"]
    f_write = kib / write["copy"]
    T = 4096
    alg = {"gemm_fwd_tensor": 2 * T * T + 2 * T * T, "gemm_dgrad_tensor": 2 * T * T + 2 * T * T,
           "gemm_wgrad_tensor": 2 * T * T + 4 * T * T,
           "cast_transpose_amax_e4m3": 4 * T * T, "cast_transpose_amax_e5m2": 4 * T * T}
    res = {"what": "HBM bytes per dispatch: FETCH_SIZE and WRITE_SIZE (KiB), each scaled by the "
                   "reading for a 256 MiB elementwise copy (neg) of known size",
           "copy_scale": {"fetch": round(f_fetch, 4), "write": round(f_write, 4)},
           "sources_sha256": sources_sha256(), "kernels": {}}
    for k in alg:
        if k not in fetch or k not in write:
            continue
        rd = fetch[k] * f_fetch * 1024.0
        wr = write[k] * f_write * 1024.0
        res["kernels"][k] = {"read_bytes": round(rd), "write_bytes": round(wr),
                             "traffic_bytes": round(rd + wr), "algorithmic_bytes": alg[k],
                             "traffic_over_algorithmic": round((rd + wr) / alg[k], 3)}
    with open(dst, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "run":
        run()
    elif len(sys.argv) >= 4 and sys.argv[1] == "summarize":
        summarize(sys.argv[2], sys.argv[3])
    else:
        print(__doc__)
        sys.exit(2)
