"""GPU parity of the power-of-two (exponent-bias) scales: scale computation,
history update and block casts bit-exact against the oracle; the GEMM with
power-of-two block operands (block scales applied inside the matrix
instruction) against the oracle's gates, on random and exactly summable
data, against the FP32-promotion path on the same inputs, and at the full
block-wise forward size on sampled outputs."""
import numpy as np
import pytest
import torch

from fp8_mixed_precision_linear_amd import datagen
from tests.gpu_util import Guarded, dev, dev_bf16, gate_stats, gemm_check, h_sampler, gemm_gate, log_gate, say
from tests.test_gpu_block_gemm import (GEMM_SHAPES, amax_of_output, narrow_codes, rand_codes,
                                       run_gemm)
from tests.test_oracle_pow2 import _amax_samples

pytestmark = pytest.mark.gpu

P2 = {1: 3, 2: 4}          # block layout code -> power-of-two code


@pytest.fixture(scope="module")
def L():
    from fp8_mixed_precision_linear_amd import lib
    assert torch.cuda.is_available()
    return lib


def bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("margin", [0, 3])
def test_compute_scale_pow2(O, L, fmt, margin):
    say("compute_scale_pow2", fmt, margin)
    a = _amax_samples(np.random.default_rng(7 + fmt))
    a = np.concatenate([a, np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 2.0 ** -149], np.float32)])
    sc, si = torch.empty(a.size, device="cuda"), torch.empty(a.size, device="cuda")
    L.fp8_compute_scale_pow2(dev(a), fmt, margin, sc, si)
    torch.cuda.synchronize()
    want = [O.compute_scale(v, fmt, margin, 1.0, pow2=True) for v in a]
    assert np.array_equal(bits(sc.cpu().numpy()), bits([w[0] for w in want]))
    assert np.array_equal(bits(si.cpu().numpy()), bits([w[1] for w in want]))


@pytest.mark.parametrize("ln,algo", [(16, 0), (16, 1), (65, 0)])
def test_history_update_pow2(O, L, ln, algo):
    say("history_pow2", ln, algo)
    rng = np.random.default_rng(ln * 3 + algo)
    n, steps = 4, 40
    am = np.abs(rng.standard_normal((steps, n))).astype(np.float32) * np.float32(10)
    am[3, 0] = 1000.0
    am[:4, 1] = 0.0
    am[7, 2] = np.nan
    am[11:, 3] = 2.0 ** -140
    for fmt in (0, 1):
        h = np.zeros((n, ln), np.float32)
        s = np.ones(n, np.float32)
        si = np.ones(n, np.float32)
        hd, sd, sid = dev(h), dev(s), dev(si)
        for t in range(steps):
            L.fp8_amax_history_update_pow2(hd, dev(am[t]), fmt, 0, algo, sd, sid)
            O.history_update(h, am[t], fmt, 0, algo, s, si, pow2=True)
            torch.cuda.synchronize()
            assert np.array_equal(bits(hd.cpu().numpy()), bits(h)), t
            assert np.array_equal(bits(sd.cpu().numpy()), bits(s)), t
            assert np.array_equal(bits(sid.cpu().numpy()), bits(si)), t


@pytest.mark.parametrize("shape", [(256, 384), (200, 300), (129, 1), (16, 16), (384, 1024)])
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("tile", [1, 2])
def test_cast_block_pow2(O, L, shape, fmt, tile):
    say("cast_block_pow2", shape, fmt, tile)
    rows, cols = shape
    rng = np.random.default_rng(rows * 13 + cols + fmt + 7 * tile)
    x = datagen.student_t3(rng, shape, 1.0)
    if x.size > 300:
        x[min(rows - 1, 5), :] = 0
        x[:, 0] = datagen.bf16_bits(np.float32(1e-30) * np.ones(rows, np.float32))   # tiny column
    nrb, ncb = (rows + 127) // 128, (cols + 127) // 128
    sshape, tshape = ((ncb, rows), (nrb, cols)) if tile == 1 else ((ncb, nrb), (nrb, ncb))
    y, s = Guarded(shape, torch.uint8), Guarded(sshape, torch.float32)
    yt, st = Guarded(shape[::-1], torch.uint8), Guarded(tshape, torch.float32)
    L.fp8_cast_block_pow2(dev_bf16(x), fmt, tile, y=y.t, scale_inv=s.t, y_t=yt.t, scale_inv_t=st.t)
    torch.cuda.synchronize()
    for g in (y, s, yt, st):
        g.check()
    ref = O.cast_block(x, fmt, tile, want_y=True, want_t=True, pow2=True)
    assert np.array_equal(y.np(), ref["y"])
    assert np.array_equal(bits(s.np()), bits(ref["sinv"]))
    assert np.array_equal(yt.np(), ref["y_t"])
    assert np.array_equal(bits(st.np()), bits(ref["sinv_t"]))


def pow2_scales(rng, scaling, rows, K, lo=-20, hi=10):
    nkb = (K + 127) // 128
    if scaling == 0:
        return np.array([rng.uniform(0.001, 2.0)], np.float32)     # any binary32 tensor scale
    shape = (nkb, rows) if scaling == 1 else (nkb, (rows + 127) // 128)
    return np.exp2(rng.integers(lo, hi + 1, shape)).astype(np.float32)


MODES_P2 = [(1, 2), (1, 1), (2, 2), (0, 2), (1, 0), (2, 1)]


@pytest.mark.parametrize("shape", GEMM_SHAPES)
@pytest.mark.parametrize("mode", MODES_P2)
@pytest.mark.parametrize("fmts", [(0, 0), (1, 0), (0, 1)])
@pytest.mark.parametrize("out_f32", [False, True])
def test_gemm_pow2_random_codes(O, L, shape, mode, fmts, out_f32):
    M, N, K = shape
    af, bf = fmts
    asc, bsc = mode
    say("gemm pow2", shape, mode, fmts, out_f32)
    rng = np.random.default_rng(M * 3 + N * 7 + K + 11 * asc + bsc + 5 * af + bf)
    A = rand_codes(rng, (M, K), af)
    B = rand_codes(rng, (N, K), bf)
    sa = pow2_scales(rng, asc, M, K)
    sb = pow2_scales(rng, bsc, N, K)
    G, raw, am = run_gemm(L, A, af, P2.get(asc, asc), sa, B, bf, P2.get(bsc, bsc), sb, out_f32)
    ref = O.gemm(A, af, asc, sa, B, bf, bsc, sb, want=("E", "F", "D", "H"))
    ok1, ok2, m1, m2 = gemm_check(G, ref, K, bf16=not out_f32)
    assert ok1 and ok2, f"componentwise rel {m1:.3e}, model-bound ratio {m2:.3f}"
    assert bits(am) == bits(amax_of_output(raw, out_f32))


@pytest.mark.parametrize("shape", GEMM_SHAPES)
@pytest.mark.parametrize("mode", [(1, 2), (1, 1), (2, 2)])
@pytest.mark.parametrize("out_f32", [False, True])
def test_gemm_pow2_exact_band_strict(O, L, shape, mode, out_f32):
    """Exactly summable data with power-of-two block scales over 31 binades:
    the strict gate holds, and the instruction-scaled result equals the
    FP32-promotion path's to within binary32 roundings of the accumulator."""
    M, N, K = shape
    asc, bsc = mode
    say("gemm pow2 strict", shape, mode, out_f32)
    rng = np.random.default_rng(M * 17 + N + K * 3 + asc + 5 * bsc)
    A = narrow_codes(rng, (M, K), 0)
    B = narrow_codes(rng, (N, K), 1)
    sa = pow2_scales(rng, asc, M, K)
    sb = pow2_scales(rng, bsc, N, K)
    G, raw, am = run_gemm(L, A, 0, P2[asc], sa, B, 1, P2[bsc], sb, out_f32)
    ref = O.gemm(A, 0, asc, sa, B, 1, bsc, sb, want=("E", "F", "D", "H"))
    ok, mx, nfl = gemm_gate(G, ref["F"], ref["D"], bf16=not out_f32)
    assert ok, f"max rel err {mx} (floored {nfl})"
    Gp, _, _ = run_gemm(L, A, 0, asc, sa, B, 1, bsc, sb, True, amax=False)
    if out_f32:
        D = ref["D"]
        assert np.all(np.abs(G.astype(np.float64) - Gp) <= 2.0 ** -20 * D + 1e-30)


def test_block_forward_pow2_full_size(O, L):
    """Block-wise forward at 8192 x 4096 x 14336 with power-of-two scales:
    casts bit-exact on sampled rows, GEMM on 128 sampled rows x 128 columns
    (every K block) under the GEMM gate |G - F| <= 1e-3 max(|F|, D/64) (+ the
    matrix unit's in-instruction bound H, see gate_stats)."""
    from fp8_mixed_precision_linear_amd import datagen as dg
    T, DI, DO = 8192, 4096, 14336
    c3 = dg.config3()
    x, w = c3["x"], c3["w"]
    xq = torch.empty((T, DI), dtype=torch.uint8, device="cuda")
    sx = torch.empty((DI // 128, T), device="cuda")
    wtq = torch.empty((DO, DI), dtype=torch.uint8, device="cuda")
    swt = torch.empty((DI // 128, DO // 128), device="cuda")
    wq = torch.empty((DI, DO), dtype=torch.uint8, device="cuda")
    sw = torch.empty((DO // 128, DI // 128), device="cuda")
    say("pow2 full-size casts")
    L.fp8_cast_block_pow2(dev_bf16(x), 0, 1, y=xq, scale_inv=sx)
    L.fp8_cast_block_pow2(dev_bf16(w), 0, 2, y=wq, scale_inv=sw, y_t=wtq, scale_inv_t=swt)
    y = torch.empty((T, DO), dtype=torch.bfloat16, device="cuda")
    say("pow2 full-size gemm")
    L.fp8_scaled_gemm(xq, 0, 3, sx, wtq, 0, 4, swt, y)
    torch.cuda.synchronize()
    rng = np.random.default_rng(99)
    rows = np.sort(rng.choice(T, 128, replace=False))
    cols = np.sort(rng.choice(DO, 128, replace=False))
    xs = np.ascontiguousarray(x[rows])
    rx = O.cast_block(xs, 0, 1, want_y=True, pow2=True)
    assert np.array_equal(xq.cpu().numpy()[rows], rx["y"])
    assert np.array_equal(bits(sx.cpu().numpy()[:, rows]), bits(rx["sinv"]))
    rw = O.cast_block(w, 0, 2, want_y=True, want_t=True, pow2=True)
    assert np.array_equal(wq.cpu().numpy(), rw["y"])
    assert np.array_equal(bits(swt.cpu().numpy()), bits(rw["sinv_t"]))
    Bsel = np.ascontiguousarray(rw["y_t"][cols])
    # the oracle on the sampled rows and columns; the 128x128 B scales of the
    # sampled columns are given per column (1x128 layout), the same values
    sb_cols = np.ascontiguousarray(np.take(rw["sinv_t"], cols // 128, axis=1))
    sxs = sx.cpu().numpy()[:, rows].copy()
    ref = O.gemm(rx["y"], 0, 1, sxs, Bsel, 0, 1, sb_cols, want=("E", "F", "D"))
    G = y.float().cpu().numpy()[np.ix_(rows, cols)]
    st = gate_stats(G, ref, bf16=True, h_of=h_sampler(O, rx["y"], 0, 1, sxs, Bsel, 0, 1, sb_cols))
    log_gate("pow2 block fwd 8192x14336x4096", st)
    assert st["max_rel_hw"] <= 1e-3, st
