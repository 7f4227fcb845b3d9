"""Pins of the oracle's row-wise scaling: the row-wise cast against numpy row
and column maxima and torch's RNE conversion; the GEMM with per-row scales
against exact rational arithmetic, the per-tensor mode (equal row scales)
and the FP32-accumulation bound."""
from fractions import Fraction

import numpy as np
import pytest

from fp8_mixed_precision_linear_amd import datagen
from tests.test_oracle_gemm import frac_decode, rand_codes
from tests.test_oracle_scaling import FMAX, lib_cast


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("shape", [(64, 384), (37, 129), (1, 5), (200, 1)])
def test_cast_rowwise_vs_library(O, fmt, shape):
    rng = np.random.default_rng(sum(shape) + fmt)
    x = datagen.student_t3(rng, shape, 1.0)
    rows, cols = shape
    if rows > 2:
        x[1, :] = 0                                    # an all-zero row: scale 1
    xf = datagen.bf16_to_f32(x)
    got = O.cast_rowwise(x, fmt, want_y=True, want_t=True)
    for r in range(rows):
        am = np.max(np.abs(xf[r]))
        s = np.float32(FMAX[fmt]) / am if am > 0 else np.float32(1.0)
        assert got["sinv"][r] == np.float32(1.0) / s
        assert np.array_equal(got["y"][r], lib_cast(x[r], s, fmt))
    xt = np.ascontiguousarray(x.T)
    for c in range(cols):
        am = np.max(np.abs(xf[:, c]))
        s = np.float32(FMAX[fmt]) / am if am > 0 else np.float32(1.0)
        assert got["sinv_t"][c] == np.float32(1.0) / s
        assert np.array_equal(got["y_t"][c], lib_cast(xt[c], s, fmt))


def _row_exact(A, af, sa, B, bf, sb):
    M, K = A.shape
    N = B.shape[0]
    out = np.empty((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            tot = sum((frac_decode(int(A[m, k]), af) * frac_decode(int(B[n, k]), bf)
                       for k in range(K)), Fraction(0))
            out[m, n] = tot * Fraction(float(sa[m])) * Fraction(float(sb[n]))
    return out


@pytest.mark.parametrize("asc,bsc", [(5, 5), (5, 0), (0, 5)])
def test_rowwise_gemm_exact(O, asc, bsc):
    rng = np.random.default_rng(11 + asc + 2 * bsc)
    M, N, K = 3, 4, 256
    A = rand_codes(rng, (M, K), 0)
    B = rand_codes(rng, (N, K), 1)
    sa = np.exp2(rng.uniform(-8, 4, M)).astype(np.float32) if asc == 5 else np.float32([0.37])
    sb = np.exp2(rng.uniform(-8, 4, N)).astype(np.float32) if bsc == 5 else np.float32([1.9])
    ref = O.gemm(A, 0, asc, sa, B, 1, bsc, sb)
    ex = _row_exact(A, 0, np.broadcast_to(sa, (M,)), B, 1, np.broadcast_to(sb, (N,)))
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(float(ref["E"][m, n])) - ex[m, n]) <= abs(ex[m, n]) * Fraction(1, 2 ** 52)


def test_rowwise_equal_scales_is_tensor_mode(O):
    rng = np.random.default_rng(5)
    M, N, K = 40, 24, 384
    A = rand_codes(rng, (M, K), 0)
    B = rand_codes(rng, (N, K), 0)
    t = O.gemm(A, 0, 0, np.float32([0.75]), B, 0, 0, np.float32([1.5]))
    r = O.gemm(A, 0, 5, np.full(M, 0.75, np.float32), B, 0, 5, np.full(N, 1.5, np.float32))
    for k in ("E", "F", "D"):
        assert np.array_equal(t[k], r[k])


def test_rowwise_f32_accumulation_within_bound(O):
    rng = np.random.default_rng(9)
    M, N, K = 32, 32, 1024
    A = rand_codes(rng, (M, K), 0)
    B = rand_codes(rng, (N, K), 1)
    sa = np.exp2(rng.uniform(-10, 2, M)).astype(np.float32)
    sb = np.exp2(rng.uniform(-10, 2, N)).astype(np.float32)
    ref = O.gemm(A, 0, 5, sa, B, 1, 5, sb)
    j = K / 128 + 3
    gam = j * 2.0 ** -24 / (1 - j * 2.0 ** -24)
    assert np.all(np.abs(ref["F"].astype(np.float64) - ref["E"]) <= gam * ref["D"] + 1e-300)
    # scaling by the row scales afterwards: F is fl32(fl32(acc sa) sb) of the per-tensor F
    one = O.gemm(A, 0, 0, np.float32([1.0]), B, 1, 0, np.float32([1.0]))
    want = (one["F"] * sa[:, None]).astype(np.float32) * sb[None, :]
    assert np.array_equal(ref["F"], want.astype(np.float32))
