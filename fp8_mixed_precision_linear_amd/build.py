"""Build libfp8lin.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m fp8_mixed_precision_linear_amd.build

Every .hip file under csrc/ is compiled with hipcc for gfx950 into
_build/*.o (in parallel) and linked into fp8_mixed_precision_linear_amd/
libfp8lin.so.  Packed-FP32 instruction selection is disabled for all device
code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfp8lin.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libfp8lin)")


def device_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-Wno-inline-asm", "-I", os.path.join(ROOT, "include")]


# Per-file code-generation options.  The FP32-promoted block GEMMs
# (gemm_big.hip) schedule with the compiler's max-ILP strategy: block WGRAD
# 2% faster at 8192x28672x8192, FWD / DGRAD unchanged, results identical,
# same registers and no scratch.
EXTRA_FLAGS = {"gemm_big.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose: bool = False, jobs: int = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    srcs = sources()
    jobs = jobs or max(1, min(len(srcs), os.cpu_count() or 1, 16))

    def one(src):
        obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
        cmd = [cc, *device_flags(), *EXTRA_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, flush=True)
        return obj

    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(one, srcs))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
