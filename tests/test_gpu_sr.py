"""GPU parity of stochastic rounding and the exponentially weighted amax:
  - the stochastic-rounding cast bit-exact against the oracle (codes,
    transposed copy, fused amax) on every kernel path (flat, tiled
    cast-transpose, element-wise for other shapes, the flat kernel's tail),
    on all 65,536 bf16 patterns at several scales (the FP8 subnormal branch
    included), with 64-bit seeds and offsets, and at 4096 x 4096;
  - the EWMA update bit-exact against the oracle over long sequences with
    zero, NaN and Inf amaxes, for several weights, margins and formats."""
import numpy as np
import pytest
import torch

from fp8_mixed_precision_linear_amd import datagen
from tests.gpu_util import Guarded, dev, dev_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    from fp8_mixed_precision_linear_amd import lib
    assert torch.cuda.is_available()
    return lib


def bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def run_sr(L, x, fmt, s, seed, offset, want_y=True, want_t=False, amax=False):
    rows, cols = x.shape
    y = Guarded((rows, cols), torch.uint8) if want_y else None
    yt = Guarded((cols, rows), torch.uint8) if want_t else None
    am = Guarded((1,), torch.float32) if amax else None
    L.fp8_cast_sr(dev_bf16(x), fmt, dev(np.array([s], np.float32)), seed, offset,
                  y=y.t if y else None, y_t=yt.t if yt else None, amax_out=am.t if am else None)
    torch.cuda.synchronize()
    for g in (y, yt, am):
        if g is not None:
            g.check()
    return (y.np() if y else None, yt.np() if yt else None, am.np()[0] if am else None)


SHAPES = [(256, 384), (64, 4096), (200, 300), (33, 17), (1, 1), (5, 1000), (1024, 16)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("want", ["y", "t", "both"])
def test_cast_sr(O, L, shape, fmt, want):
    rows, cols = shape
    say("cast_sr", shape, fmt, want)
    rng = np.random.default_rng(rows * 7 + cols + fmt)
    x = datagen.student_t3(rng, shape, 1.0)
    if x.size > 64:
        flat = x.reshape(-1)
        flat[3] = datagen.bf16_bits(np.float32([np.inf]))[0]
        flat[10] = datagen.bf16_bits(np.float32([-np.nan]))[0]
        flat[20] = 0x8000                                    # -0
        flat[30:40] = datagen.bf16_bits(np.float32(2.0 ** -12) * np.arange(1, 11, dtype=np.float32))
    s = 40.0 if fmt == 0 else 3000.0
    seed, off = 0x9E3779B97F4A7C15 + rows, 0xFFFFFFFF00000000 + cols
    wy, wt = want in ("y", "both"), want in ("t", "both")
    y, yt, am = run_sr(L, x, fmt, s, seed, off, wy, wt, amax=True)
    ry, ryt = O.cast_sr(x, s, fmt, seed, off, want_y=wy, want_t=wt)
    if wy:
        assert np.array_equal(y, ry)
    if wt:
        assert np.array_equal(yt, ryt)
    assert bits(am) == bits(O.amax(x))


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("scale", [1.0, 2.0 ** -10, 3.0, 2.0 ** 20, 1e-30])
def test_cast_sr_all_bf16(O, L, fmt, scale):
    say("cast_sr all bf16", fmt, scale)
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    for seed, off in ((1, 0), (2 ** 64 - 1, 2 ** 63 + 12345)):
        y, yt, _ = run_sr(L, x, fmt, scale, seed, off, True, True)
        ry, _ = O.cast_sr(x, scale, fmt, seed, off)
        assert np.array_equal(y, ry)
        assert np.array_equal(yt, ry.T)


def test_cast_sr_full_size(O, L):
    """dY at 4096 x 4096 (the delayed-scaling workload, step 0) as E5M2 with
    the transposed copy: every code bit-exact; and unbiased on average."""
    say("cast_sr full size")
    dy = datagen.config2_step(0)["dy"]
    s = 2.0 ** 20
    y, yt, am = run_sr(L, dy, 1, s, 42, 7, True, True, amax=True)
    ry, _ = O.cast_sr(dy, s, 1, 42, 7)
    assert np.array_equal(y, ry)
    assert np.array_equal(yt, ry.T)
    v = datagen.bf16_to_f32(dy).astype(np.float64) * s
    q = O.decode(y.reshape(-1), 1).reshape(y.shape)
    rn = O.decode(O.encode(v.astype(np.float32).reshape(-1), 1), 1).reshape(y.shape)
    # the mean rounding error of SR is within a few standard errors of zero;
    # round-to-nearest shows the same data's deterministic error for scale
    err = q - v
    se = np.sqrt(np.mean(err ** 2) / err.size)
    assert abs(np.mean(err)) < 6 * se, (np.mean(err), se, np.mean(rn - v))


@pytest.mark.parametrize("beta", [0.0, 0.5, 0.9, 0.999, 1.0])
@pytest.mark.parametrize("fmt,margin", [(0, 0), (1, 0), (0, 3)])
def test_ewma_update(O, L, beta, fmt, margin):
    say("ewma", beta, fmt, margin)
    rng = np.random.default_rng(int(beta * 1000) + 10 * fmt + margin)
    n, steps = 5, 60
    am = np.abs(rng.standard_normal((steps, n))).astype(np.float32) * np.float32(30)
    am[5, 0] = 1e4
    am[:3, 1] = 0.0
    am[7, 2] = np.nan
    am[9, 3] = np.inf
    am[20:, 4] = 2.0 ** -130
    e, s, si = np.zeros(n, np.float32), np.ones(n, np.float32), np.ones(n, np.float32)
    ed, sd, sid = dev(e), dev(s), dev(si)
    for t in range(steps):
        L.fp8_amax_ewma_update(ed, dev(am[t]), beta, fmt, margin, sd, sid)
        O.amax_ewma_update(e, am[t], beta, fmt, margin, s, si)
        torch.cuda.synchronize()
        assert np.array_equal(bits(ed.cpu().numpy()), bits(e)), t
        assert np.array_equal(bits(sd.cpu().numpy()), bits(s)), t
        assert np.array_equal(bits(sid.cpu().numpy()), bits(si)), t


# ------------------------------------------- generator state on the device ---
def _state(seed, offset):
    """int64 tensor holding two unsigned 64-bit words (seed, offset)."""
    w = np.array([seed, offset], np.uint64).view(np.int64)
    return torch.from_numpy(w.copy()).cuda()


@pytest.mark.parametrize("shape", [(256, 384), (33, 17), (4096, 4096)])
@pytest.mark.parametrize("fmt", [0, 1])
def test_cast_sr_state_equals_by_value_call(O, L, shape, fmt):
    """Seed and offset read on the device give the codes of the by-value
    call (every kernel path), and the offset then moves on by `advance`."""
    rows, cols = shape
    say("cast_sr_state", shape, fmt)
    rng = np.random.default_rng(rows + 3 * cols + fmt)
    x = datagen.normal(rng, shape, 1e-3)
    s = 448.0 / 4e-3 if fmt == 0 else 57344.0 / 4e-3
    seed, offset = 0xDEADBEEF12345678, (1 << 40) + 7
    want_y, want_t, want_am = run_sr(L, x, fmt, s, seed, offset, want_y=True, want_t=True, amax=True)
    st = _state(seed, offset)
    y, yt, am = Guarded(shape, torch.uint8), Guarded(shape[::-1], torch.uint8), Guarded((1,), torch.float32)
    L.fp8_cast_sr_state(dev_bf16(x), fmt, dev(np.array([s], np.float32)), st, 5,
                        y=y.t, y_t=yt.t, amax_out=am.t)
    torch.cuda.synchronize()
    for g in (y, yt, am):
        g.check()
    assert np.array_equal(y.np(), want_y) and np.array_equal(yt.np(), want_t)
    assert bits(am.np()[0]) == bits(want_am)
    got = st.cpu().numpy().view(np.uint64)
    assert int(got[0]) == seed and int(got[1]) == offset + 5
    if rows * cols <= 1 << 17:   # the oracle on the small shapes
        ry, _ = O.cast_sr(x, np.float32(s), fmt, seed, offset, want_y=True)
        assert np.array_equal(y.np(), ry)


def test_cast_sr_state_graph_replays_draw_fresh_words(O, L):
    """One stochastic-rounding cast captured in a HIP graph and replayed
    three times (host reads between replays): replay k uses offset0 + k,
    each replay's codes equal the oracle's at that offset, and they differ."""
    say("cast_sr_state graph")
    rng = np.random.default_rng(5)
    shape = (512, 768)
    x = datagen.normal(rng, shape, 1e-3)
    s = np.float32(57344.0 / 5e-3)
    seed, off0 = 1234, 99
    xd, sd = dev_bf16(x), dev(np.array([s], np.float32))
    st = _state(seed, off0)
    y = torch.empty(shape, dtype=torch.uint8, device="cuda")
    yt = torch.empty(shape[::-1], dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.fp8_cast_sr_state(xd, 1, sd, st, 1, y=y, y_t=yt)
    torch.cuda.synchronize()
    st.copy_(_state(seed, off0))      # capture ran nothing; start from off0
    torch.cuda.synchronize()
    outs = []
    for k in range(3):
        g.replay()
        torch.cuda.synchronize()
        got, got_t = y.cpu().numpy(), yt.cpu().numpy()
        ry, rt = O.cast_sr(x, s, 1, seed, off0 + k, want_y=True, want_t=True)
        assert np.array_equal(got, ry), k
        assert np.array_equal(got_t, rt), k
        assert int(st.cpu().numpy().view(np.uint64)[1]) == off0 + k + 1
        outs.append(got)
    assert not np.array_equal(outs[0], outs[1]) and not np.array_equal(outs[1], outs[2])
    del g
