"""GPU parity of per-row (per-channel) scaling:
  - the row-wise cast bit-exact against the oracle (codes and inverse
    scales, row-major copy with row scales and transposed copy with column
    scales), on every kernel path: row lengths up to 4096, 8192, 16384 and
    32768 columns, the element-wise path for other shapes, several rows per
    workgroup, all-zero, Inf and NaN rows and columns;
  - the GEMM with per-row scales (per-row x per-row, per-row x per-tensor)
    against the oracle's gates, with an FP8 output, and on the small-tile
    kernel (K beyond the large-tile kernel's scale table);
  - the row-wise forward, dgrad and wgrad at 4096 x 4096 x 4096 (the
    delayed-scaling workload's shapes and data) on sampled outputs."""
import numpy as np
import pytest
import torch

from fp8_mixed_precision_linear_amd import datagen
from tests.gpu_util import Guarded, dev, dev_bf16, gemm_check, say
from tests.test_gpu_block_gemm import GEMM_SHAPES, amax_of_output, rand_codes, run_gemm
from tests.test_gpu_configs import check_gemm_sampled

pytestmark = pytest.mark.gpu

ROW = 5


@pytest.fixture(scope="module")
def L():
    from fp8_mixed_precision_linear_amd import lib
    assert torch.cuda.is_available()
    return lib


def bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def special_input(rng, rows, cols):
    x = datagen.student_t3(rng, (rows, cols), 1.0)
    if rows >= 6 and cols >= 6:
        x[1, :] = 0                                             # all-zero row
        x[:, 2] = 0                                             # all-zero column
        x[3, 4] = datagen.bf16_bits(np.float32([np.inf]))[0]    # Inf: its row and column fall back
        x[4, 5] = datagen.bf16_bits(np.float32([np.nan]))[0]    # NaN likewise
        x[:, 0] = datagen.bf16_bits(np.float32(1e-30) * np.ones(rows, np.float32))  # tiny column
    return x


CAST_SHAPES = [(64, 384), (200, 4096), (128, 8192), (48, 16384), (80, 16384), (64, 32768),
               (32, 32768), (16, 40000), (33, 100), (1, 8), (4096, 16), (4112, 256)]


@pytest.mark.parametrize("shape", CAST_SHAPES)
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("want", ["y", "t", "both"])
def test_cast_rowwise(O, L, shape, fmt, want):
    rows, cols = shape
    say("cast_rowwise", shape, fmt, want)
    rng = np.random.default_rng(rows * 31 + cols + 7 * fmt)
    x = special_input(rng, rows, cols)
    wy, wt = want in ("y", "both"), want in ("t", "both")
    y = Guarded((rows, cols), torch.uint8) if wy else None
    s = Guarded((rows,), torch.float32) if wy else None
    yt = Guarded((cols, rows), torch.uint8) if wt else None
    st = Guarded((cols,), torch.float32) if wt else None
    L.fp8_cast_rowwise(dev_bf16(x), fmt, y=y.t if wy else None, scale_inv=s.t if wy else None,
                       y_t=yt.t if wt else None, scale_inv_t=st.t if wt else None)
    torch.cuda.synchronize()
    ref = O.cast_rowwise(x, fmt, want_y=wy, want_t=wt)
    if wy:
        y.check(); s.check()
        assert np.array_equal(bits(s.np()), bits(ref["sinv"]))
        assert np.array_equal(y.np(), ref["y"])
    if wt:
        yt.check(); st.check()
        assert np.array_equal(bits(st.np()), bits(ref["sinv_t"]))
        assert np.array_equal(yt.np(), ref["y_t"])


def test_cast_rowwise_repeated_calls(O, L):
    """Partial column maxima live in y_t and scale_inv_t during the call: a
    second call on new data into the same buffers starts afresh."""
    rows, cols = 256, 512
    outs = (torch.empty((rows, cols), dtype=torch.uint8, device="cuda"),
            torch.empty(rows, device="cuda"),
            torch.empty((cols, rows), dtype=torch.uint8, device="cuda"),
            torch.empty(cols, device="cuda"))
    for seed in (1, 2):
        say("cast_rowwise repeated", seed)
        x = datagen.normal(np.random.default_rng(seed), (rows, cols), 10.0 if seed == 1 else 0.01)
        L.fp8_cast_rowwise(dev_bf16(x), 0, *outs)
        torch.cuda.synchronize()
        ref = O.cast_rowwise(x, 0, want_y=True, want_t=True)
        assert np.array_equal(outs[0].cpu().numpy(), ref["y"])
        assert np.array_equal(bits(outs[1].cpu().numpy()), bits(ref["sinv"]))
        assert np.array_equal(outs[2].cpu().numpy(), ref["y_t"])
        assert np.array_equal(bits(outs[3].cpu().numpy()), bits(ref["sinv_t"]))


def row_scales(rng, scaling, rows):
    if scaling == 0:
        return np.array([rng.uniform(0.001, 2.0)], np.float32)
    return np.exp2(rng.uniform(-12, 4, rows)).astype(np.float32)


@pytest.mark.parametrize("shape", GEMM_SHAPES)
@pytest.mark.parametrize("mode", [(ROW, ROW), (ROW, 0), (0, ROW)])
@pytest.mark.parametrize("fmts", [(0, 0), (1, 0), (0, 1)])
@pytest.mark.parametrize("out_f32", [False, True])
def test_gemm_rowwise(O, L, shape, mode, fmts, out_f32):
    M, N, K = shape
    af, bf = fmts
    asc, bsc = mode
    say("gemm rowwise", shape, mode, fmts, out_f32)
    rng = np.random.default_rng(M * 5 + N * 11 + K + 3 * asc + bsc + 7 * af + bf)
    A = rand_codes(rng, (M, K), af)
    B = rand_codes(rng, (N, K), bf)
    sa = row_scales(rng, asc, M)
    sb = row_scales(rng, bsc, N)
    G, raw, am = run_gemm(L, A, af, asc, sa, B, bf, bsc, sb, out_f32)
    ref = O.gemm(A, af, asc, sa, B, bf, bsc, sb, want=("E", "F", "D", "H"))
    ok1, ok2, m1, m2 = gemm_check(G, ref, K, bf16=not out_f32)
    assert ok1 and ok2, f"componentwise rel {m1:.3e}, model-bound ratio {m2:.3f}"
    assert bits(am) == bits(amax_of_output(raw, out_f32))


@pytest.mark.parametrize("shape", [(256, 512, 384), (200, 136, 384), (129, 257, 256)])
@pytest.mark.parametrize("out_fmt", [0, 1])
def test_gemm_rowwise_fp8_output(O, L, shape, out_fmt):
    M, N, K = shape
    say("gemm rowwise fp8 out", shape, out_fmt)
    rng = np.random.default_rng(M + 5 * N + K + out_fmt)
    A = rand_codes(rng, (M, K), 0)
    B = rand_codes(rng, (N, K), 1)
    sa, sb = row_scales(rng, ROW, M), row_scales(rng, ROW, N)
    D32 = Guarded((M, N), torch.float32)
    L.fp8_scaled_gemm(dev(A), 0, ROW, dev(sa), dev(B), 1, ROW, dev(sb), D32.t)
    torch.cuda.synchronize()
    D32.check()
    G = D32.np()
    ref = O.gemm(A, 0, ROW, sa, B, 1, ROW, sb, want=("E", "F", "D", "H"))
    ok1, ok2, m1, m2 = gemm_check(G, ref, K, bf16=False)
    assert ok1 and ok2, f"componentwise rel {m1:.3e}, model-bound ratio {m2:.3f}"
    fmax = 448.0 if out_fmt == 0 else 57344.0
    s_out = np.float32(fmax / max(np.quantile(np.abs(G), 0.95), 1e-30))
    D8, Dt, am = Guarded((M, N), torch.uint8), Guarded((N, M), torch.uint8), Guarded((1,), torch.float32)
    L.fp8_scaled_gemm(dev(A), 0, ROW, dev(sa), dev(B), 1, ROW, dev(sb), D8.t, d_amax=am.t,
                      d_scale=dev(np.array([s_out], np.float32)), d_fmt=out_fmt, D_t=Dt.t)
    torch.cuda.synchronize()
    D8.check(); Dt.check(); am.check()
    want = O.encode((G * s_out).astype(np.float32), out_fmt).reshape(M, N)
    assert np.array_equal(D8.np(), want)
    assert np.array_equal(Dt.np(), want.T)
    assert bits(am.np()[0]) == bits(np.max(np.abs(G)))


@pytest.mark.parametrize("mode", [(ROW, ROW), (0, 0), (1, 2)])
@pytest.mark.parametrize("K", [65536, 65536 + 256])
def test_gemm_long_k(O, L, mode, K):
    """K = 65536 is the large-tile kernel's last size (512 K blocks of scale
    table); beyond it the small-tile kernel runs: tensor, per-row and block
    modes on both."""
    M, N = 40, 72
    asc, bsc = mode
    say("gemm long K", mode, K)
    rng = np.random.default_rng(K + 3 * asc + bsc)
    A = rand_codes(rng, (M, K), 0)
    B = rand_codes(rng, (N, K), 1)
    nkb = (K + 127) // 128
    if asc == ROW:
        sa, sb = row_scales(rng, ROW, M), row_scales(rng, ROW, N)
    elif asc == 0:
        sa, sb = row_scales(rng, 0, M), row_scales(rng, 0, N)
    else:
        sa = np.exp2(rng.uniform(-12, 4, (nkb, M))).astype(np.float32)
        sb = np.exp2(rng.uniform(-12, 4, (nkb, 1))).astype(np.float32)
    G, raw, am = run_gemm(L, A, 0, asc, sa, B, 1, bsc, sb, True)
    ref = O.gemm(A, 0, asc, sa, B, 1, bsc, sb, want=("E", "F", "D", "H"))
    ok1, ok2, m1, m2 = gemm_check(G, ref, K, bf16=False)
    assert ok1 and ok2, f"componentwise rel {m1:.3e}, model-bound ratio {m2:.3f}"
    assert bits(am) == bits(amax_of_output(raw, True))


def test_rowwise_fwd_bwd_full_size(O, L):
    """Row-wise forward, dgrad and wgrad at 4096 x 4096 x 4096 on the
    delayed-scaling workload's step-0 data: every cast bit-exact, GEMMs on
    128 sampled rows and 128 sampled columns."""
    d = datagen.config2_step(0)
    x, w, dy = d["x"], d["w"], d["dy"]
    T, DI = x.shape
    DO = w.shape[1]
    u8 = dict(dtype=torch.uint8, device="cuda")
    c = {}
    for name, a, fmt in (("x", x, 0), ("w", w, 0), ("dy", dy, 1)):
        r, k = a.shape
        c[name] = (torch.empty((r, k), **u8), torch.empty(r, device="cuda"),
                   torch.empty((k, r), **u8), torch.empty(k, device="cuda"))
        say("rowwise full-size cast", name)
        L.fp8_cast_rowwise(dev_bf16(a), fmt, *c[name])
    y = torch.empty((T, DO), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((T, DI), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((DI, DO), dtype=torch.float32, device="cuda")
    xq, sx, xtq, sxt = c["x"]
    wq, sw, wtq, swt = c["w"]
    dyq, sdy, dytq, sdyt = c["dy"]
    say("rowwise full-size gemms")
    L.fp8_scaled_gemm(xq, 0, ROW, sx, wtq, 0, ROW, swt, y)         # Y  = X W
    L.fp8_scaled_gemm(dyq, 1, ROW, sdy, wq, 0, ROW, sw, dx)        # dX = dY W^T
    L.fp8_scaled_gemm(xtq, 0, ROW, sxt, dytq, 1, ROW, sdyt, dw)    # dW = X^T dY
    torch.cuda.synchronize()
    ref = {}
    for name, a, fmt in (("x", x, 0), ("w", w, 0), ("dy", dy, 1)):
        say("rowwise full-size oracle cast", name)
        ref[name] = O.cast_rowwise(a, fmt, want_y=True, want_t=True)
        q, s, qt, st = (t.cpu().numpy() for t in c[name])
        assert np.array_equal(q, ref[name]["y"]), name
        assert np.array_equal(bits(s), bits(ref[name]["sinv"])), name
        assert np.array_equal(qt, ref[name]["y_t"]), name
        assert np.array_equal(bits(st), bits(ref[name]["sinv_t"])), name
    rx, rw, rd = ref["x"], ref["w"], ref["dy"]
    say("rowwise full-size fwd")
    check_gemm_sampled(O, y, rx["y"], 0, ROW, rx["sinv"], rw["y_t"], 0, ROW, rw["sinv_t"], True, 61,
                       a16=x, b16=np.ascontiguousarray(w.T), label="rowwise 4096 fwd")
    say("rowwise full-size dgrad")
    check_gemm_sampled(O, dx, rd["y"], 1, ROW, rd["sinv"], rw["y"], 0, ROW, rw["sinv"], True, 62,
                       a16=dy, b16=w, label="rowwise 4096 dgrad")
    say("rowwise full-size wgrad")
    check_gemm_sampled(O, dw, rx["y_t"], 0, ROW, rx["sinv_t"], rd["y_t"], 1, ROW, rd["sinv_t"], False,
                       63, a16=np.ascontiguousarray(x.T), b16=np.ascontiguousarray(dy.T),
                       label="rowwise 4096 wgrad")
