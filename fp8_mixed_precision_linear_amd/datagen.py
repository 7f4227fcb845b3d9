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

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "bf16_bits", "bf16_to_f32", "normal", "student_t3", "with_outlier_columns",
    "config1", "config2_step", "config3", "config4_dy", "config5_linear",
    "config5_outlier_cols", "chunked_rows", "C5_LINEARS",
]

_CHUNK_ROWS = 1024


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round binary32 values to bf16 (nearest, ties to even) -> uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32)
    # 32-bit arithmetic, in place: only NaN patterns can wrap, and those are
    # replaced below
    r = b >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += b
    r >>= np.uint32(16)
    r = r.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = ((b[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
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
        t = rng.standard_normal((r1 - r0, cols), dtype=np.float32)      # z0
        den = rng.standard_normal((r1 - r0, cols), dtype=np.float32)    # z1
        den *= den
        z = rng.standard_normal((r1 - r0, cols), dtype=np.float32)      # z2
        z *= z
        den += z
        rng.standard_normal((r1 - r0, cols), dtype=np.float32, out=z)   # z3
        z *= z
        den += z
        den /= np.float32(3.0)
        np.sqrt(den, out=den)
        t /= den
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


# Transformer-block linear set: name -> (in, out)
C5_LINEARS = {
    "qkv": (8192, 10240),
    "o": (8192, 8192),
    "gate": (8192, 28672),
    "up": (8192, 28672),
    "down": (28672, 8192),
}
_C5_ORDER = ["qkv", "o", "gate", "up", "down"]
_X, _W, _DY = 0, 1, 2


def _workers() -> int:
    return max(1, min(os.cpu_count() or 1, 16))


def chunked_rows(shape, seed: int, key: tuple, draw, row_range=None) -> np.ndarray:
    """bf16 bits of a [rows x cols] tensor drawn in chunks of 1024 rows, chunk
    c from its own generator default_rng(SeedSequence(seed, spawn_key=key +
    (c,))) by `draw(rng, chunk_shape)`, so chunks are independent and are
    drawn on worker threads.  `row_range` = (r0, r1) (chunk-aligned r0)
    returns only those rows, with the same values as the full tensor."""
    rows, cols = shape
    r0, r1 = (0, rows) if row_range is None else row_range
    assert r0 % _CHUNK_ROWS == 0 and 0 <= r0 <= r1 <= rows
    out = np.empty((r1 - r0, cols), dtype=np.uint16)

    def one(c):
        a = c * _CHUNK_ROWS
        b = min(rows, a + _CHUNK_ROWS, r1)
        rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=tuple(key) + (c,)))
        out[a - r0:b - r0] = draw(rng, (min(rows, a + _CHUNK_ROWS) - a, cols))[:b - a]

    chunks = range(r0 // _CHUNK_ROWS, (r1 + _CHUNK_ROWS - 1) // _CHUNK_ROWS)
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, chunks))
    return out


def config5_outlier_cols(name: str, seed: int = 0) -> np.ndarray:
    """The round(0.001 * in) outlier channels of a linear's activation
    (gate and up share theirs), from SeedSequence(seed, spawn_key=(i, 0))."""
    d_in = C5_LINEARS[name][0]
    x_idx = _C5_ORDER.index("gate") if name == "up" else _C5_ORDER.index(name)
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(x_idx, _X)))
    return np.sort(rng.choice(d_in, int(round(0.001 * d_in)), replace=False))


def config5_linear(name: str, seed: int = 0, tokens: int = 8192, token_range=None,
                   parts=("x", "w", "dy")):
    """One linear of the transformer-block set, [T x in] activation X,
    [in x out] weight W, [T x out] gradient dY:
      X  Student-t(3) with round(0.001*in) channels x100 (config5_outlier_cols);
      W  N(0, 0.02);  dY  N(0, 1e-3).
    Linear i (qkv, o, gate, up, down = 0..4) draws tensor r (X 0, W 1, dY 2)
    in chunks of 1024 rows, chunk c from SeedSequence(seed, spawn_key=(i, r,
    c)); gate and up share the activation of "gate".  `token_range` limits
    X and dY to those token rows (same values as in the full tensors)."""
    d_in, d_out = C5_LINEARS[name]
    idx = _C5_ORDER.index(name)
    x_idx = _C5_ORDER.index("gate") if name == "up" else idx
    cols = config5_outlier_cols(name, seed)
    out = {"outlier_cols": cols}
    if "x" in parts:
        out["x"] = chunked_rows((tokens, d_in), seed, (x_idx, _X),
                                lambda r, sh: student_t3(r, sh, 1.0, outlier_cols=cols,
                                                         outlier_mul=100.0),
                                token_range)
    if "w" in parts:
        out["w"] = chunked_rows((d_in, d_out), seed, (idx, _W), lambda r, sh: normal(r, sh, 0.02))
    if "dy" in parts:
        out["dy"] = chunked_rows((tokens, d_out), seed, (idx, _DY),
                                 lambda r, sh: normal(r, sh, 1e-3), token_range)
    return out
