"""Seeded synthetic inputs for the FP8 scaled linear layer.

This module is the one piece shared by the HIP path's tests/benchmark and the
CPU oracle's tests.  It holds none of the method's arithmetic: it draws
binary32 samples from numpy's PCG64 generator and rounds them to bf16 bit
patterns (the layer's input dtype), nothing else.

Workload shapes and distributions follow the configurations the layer is
measured on (per-tensor forward 256x512x512, delayed-scaling fwd+bwd 4096^3
over 16 steps, block-wise 8192x4096x14336 forward and backward, and the
transformer-block linear set at hidden 8192 / FFN 28672).  "N(0, s)" means a
normal with standard deviation s.  Weights are stored [in x out].
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits", "bf16_to_f32", "normal", "student_t3", "with_outlier_columns",
    "config1", "config2_step", "config3", "config4_dy", "config5_linear",
    "C5_LINEARS",
]

_CHUNK_ROWS = 1024


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round binary32 values to bf16 (nearest, ties to even) -> uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32).astype(np.uint64)
    nan = (b & 0x7FFFFFFF) > 0x7F800000
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = ((b[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to binary32 values (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    """bf16 bits of N(0, std) samples, drawn row-chunk by row-chunk."""
    rows, cols = shape
    out = np.empty((rows, cols), dtype=np.uint16)
    for r0 in range(0, rows, _CHUNK_ROWS):
        r1 = min(rows, r0 + _CHUNK_ROWS)
        z = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        z *= np.float32(std)
        out[r0:r1] = bf16_bits(z)
    return out


def student_t3(rng: np.random.Generator, shape, scale: float = 1.0,
               outlier_cols=None, outlier_mul: float = 1.0) -> np.ndarray:
    """bf16 bits of Student-t(3) samples: t = z0 / sqrt((z1^2+z2^2+z3^2)/3).

    Per row chunk, z0..z3 are drawn in that order as [chunk, cols] blocks.
    `outlier_cols` (if given) are multiplied by `outlier_mul` in binary32
    before the bf16 rounding.
    """
    rows, cols = shape
    out = np.empty((rows, cols), dtype=np.uint16)
    for r0 in range(0, rows, _CHUNK_ROWS):
        r1 = min(rows, r0 + _CHUNK_ROWS)
        z0 = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        z1 = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        z2 = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        z3 = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        den = np.sqrt((z1 * z1 + z2 * z2 + z3 * z3) / np.float32(3.0))
        t = z0 / den
        if scale != 1.0:
            t *= np.float32(scale)
        if outlier_cols is not None:
            t[:, outlier_cols] *= np.float32(outlier_mul)
        out[r0:r1] = bf16_bits(t)
    return out


def with_outlier_columns(rng: np.random.Generator, x_f32: np.ndarray, n_cols: int,
                         mul: float):
    """Pick `n_cols` distinct columns and multiply them by `mul` (binary32)."""
    cols = rng.choice(x_f32.shape[1], n_cols, replace=False)
    x_f32[:, cols] *= np.float32(mul)
    return cols


def config1(seed: int = 0):
    """Per-tensor current-scaling forward: X 256x512 N(0,1) with 4 outlier
    columns x50, W [512 in x 512 out] N(0,0.02).  Draw order: X, the outlier
    columns, W."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((256, 512), dtype=np.float32)
    cols = with_outlier_columns(rng, x, 4, 50.0)
    w = rng.standard_normal((512, 512), dtype=np.float32) * np.float32(0.02)
    return {"x": bf16_bits(x), "w": bf16_bits(w), "outlier_cols": np.sort(cols)}


def config2_step(step: int, seed: int = 0, tokens: int = 4096, d_in: int = 4096,
                 d_out: int = 4096):
    """Delayed-scaling fwd+bwd step `step`: generator seeded with seed+step,
    draw order X [T x in] N(0,1), W [in x out] N(0,0.02), dY [T x out]
    N(0,1e-4)."""
    rng = np.random.default_rng(seed + step)
    x = normal(rng, (tokens, d_in), 1.0)
    w = normal(rng, (d_in, d_out), 0.02)
    dy = normal(rng, (tokens, d_out), 1e-4)
    return {"x": x, "w": w, "dy": dy}


def config3(seed: int = 0, tokens: int = 8192, d_in: int = 4096, d_out: int = 14336):
    """Block-wise forward: X [T x in] Student-t(3) x1.0, W [in x out]
    N(0,0.02); one generator, draw order X then W (then config4_dy)."""
    rng = np.random.default_rng(seed)
    x = student_t3(rng, (tokens, d_in), 1.0)
    w = normal(rng, (d_in, d_out), 0.02)
    return {"x": x, "w": w, "rng": rng}


def config4_dy(rng: np.random.Generator, tokens: int = 8192, d_out: int = 14336):
    """Block-wise backward gradient dY [T x out] N(0,1e-3), drawn from the
    generator config3 returned (after X and W)."""
    return normal(rng, (tokens, d_out), 1e-3)


# Transformer-block linear set: name -> (in, out, activation input group)
C5_LINEARS = {
    "qkv": (8192, 10240),
    "o": (8192, 8192),
    "gate": (8192, 28672),
    "up": (8192, 28672),
    "down": (28672, 8192),
}
_C5_ORDER = ["qkv", "o", "gate", "up", "down"]


def config5_linear(name: str, seed: int = 0, tokens: int = 8192, scale_rows: int = None):
    """One linear of the transformer-block set.  Each linear has its own
    generator: SeedSequence(seed, spawn_key=(index,)); gate and up share the
    gate/up activation (index of "gate").  Draw order: X (Student-t(3) with
    round(0.001*in) channels x100), W [in x out] N(0,0.02), dY [T x out]
    N(0,1e-3).  `scale_rows` limits T for parity-sized runs."""
    d_in, d_out = C5_LINEARS[name]
    t = tokens if scale_rows is None else scale_rows
    idx = _C5_ORDER.index(name)
    x_idx = _C5_ORDER.index("gate") if name == "up" else idx
    rng_x = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(x_idx,)))
    n_out = int(round(0.001 * d_in))
    cols = np.sort(rng_x.choice(d_in, n_out, replace=False))
    x = student_t3(rng_x, (t, d_in), 1.0, outlier_cols=cols, outlier_mul=100.0)
    rng_w = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(idx, 1)))
    w = normal(rng_w, (d_in, d_out), 0.02)
    dy = normal(rng_w, (t, d_out), 1e-3)
    return {"x": x, "w": w, "dy": dy, "outlier_cols": cols}
