"""GPU parity: amax, compute_scale, amax-history update and the per-tensor
casts (with fused transpose and amax), bit-exact against the CPU oracle on
every element.  Calls go through the C ABI (the ctypes binding)."""
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


ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)


# ------------------------------------------------------------------ amax ---
@pytest.mark.parametrize("shape", [(0, 0), (1, 1), (1, 7), (3, 5), (256, 256), (999, 1001),
                                   (4096, 4096)])
def test_amax(O, L, shape):
    say("amax", shape)
    rng = np.random.default_rng(sum(shape))
    if shape == (256, 256):
        x = ALL_BF16.copy()
        x[(ALL_BF16 & 0x7FFF) > 0x7F80] = 0  # no NaN here (see test_amax_specials)
    else:
        x = datagen.normal(rng, shape, 3.0)
        if x.size:
            x.reshape(-1)[-1] = datagen.bf16_bits(np.array([-1234.5], np.float32))[0]
    out = Guarded((1,), torch.float32)
    L.fp8_amax(dev_bf16(x), out.t)
    torch.cuda.synchronize()
    out.check()
    assert bits(out.np())[0] == bits(O.amax(x))


def test_amax_specials(O, L):
    for special in [0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x0001, 0x8000]:
        x = np.zeros((33, 77), np.uint16)
        x[17, 5] = special
        out = torch.empty(1, dtype=torch.float32, device="cuda")
        L.fp8_amax(dev_bf16(x), out)
        torch.cuda.synchronize()
        assert bits(out.cpu().numpy())[0] == bits(O.amax(x)), hex(special)


@pytest.mark.parametrize("fmt", [0, 1])
def test_cast_stats_all_bf16_patterns(O, L, fmt):
    """Saturation / underflow counts over all 65,536 bf16 patterns (NaNs
    included) and a set of scales, equal to the oracle's (which decides
    underflow with its encoder)."""
    x = dev_bf16(ALL_BF16.reshape(256, 256))
    fmax = 448.0 if fmt == 0 else 57344.0
    for s in [1.0, 2.0 ** -12, 2.0 ** 9, 3.0, 0.7, 1e-30, fmax / 7.5, 0.0]:
        say("cast stats all-bf16", fmt, s)
        counts = torch.zeros(2, dtype=torch.int64, device="cuda")
        L.fp8_cast_stats(x, fmt, torch.tensor([s], dtype=torch.float32, device="cuda"), counts)
        torch.cuda.synchronize()
        assert tuple(counts.cpu().tolist()) == O.cast_stats(ALL_BF16, np.float32(s), fmt), s


@pytest.mark.parametrize("shape", [(33, 77), (1, 1), (257, 129), (1024, 1024), (0, 7)])
def test_cast_stats_shapes_accumulate(O, L, shape):
    """Ragged sizes (tails of n % 8 values), counts added to what the slots
    hold (two calls give twice the counts)."""
    say("cast stats", shape)
    rng = np.random.default_rng(shape[0] * 3 + shape[1])
    x = datagen.student_t3(rng, shape, 1.0) if shape[0] else np.zeros(shape, np.uint16)
    s = np.float32(60.0)
    want = O.cast_stats(x, s, 0)
    counts = torch.zeros(2, dtype=torch.int64, device="cuda")
    d = dev_bf16(x) if x.size else torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    sc = torch.tensor([s], dtype=torch.float32, device="cuda")
    L.fp8_cast_stats(d, 0, sc, counts)
    L.fp8_cast_stats(d, 0, sc, counts)
    torch.cuda.synchronize()
    assert tuple(counts.cpu().tolist()) == (2 * want[0], 2 * want[1])
    if shape == (1024, 1024):
        assert want[0] > 0 and want[1] > 0   # both rules exercised


def test_cast_stats_config1(O, L):
    """The per-tensor current-scaling forward's activation (outlier columns)
    at its own scale (448 / amax: at most the amax element itself can land
    an ulp above the max)."""
    c = datagen.config1()
    x = c["x"]
    s, _, _ = O.compute_scale(O.amax(x), 0)
    counts = torch.zeros(2, dtype=torch.int64, device="cuda")
    L.fp8_cast_stats(dev_bf16(x), 0, torch.tensor([s], dtype=torch.float32, device="cuda"), counts)
    torch.cuda.synchronize()
    got = tuple(counts.cpu().tolist())
    assert got == O.cast_stats(x, s, 0)
    assert got[0] <= 1


@pytest.mark.parametrize("shape,ld", [((512, 1024), 1024), ((33, 77), 77), ((64, 300), 512), ((0, 5), 5)])
@pytest.mark.parametrize("prior", ["below", "above", "zero"])
def test_amax_acc(O, L, shape, ld, prior):
    """fp8_amax_acc: max(prior value, max |x|) in the slot, contiguous and
    strided rows; an empty tensor leaves the slot as it was."""
    rows, cols = shape
    say("amax acc", shape, ld, prior)
    rng = np.random.default_rng(rows * 7 + ld + len(prior))
    big = datagen.normal(rng, (rows, ld), 2.0)
    view = np.ascontiguousarray(big[:, :cols])
    a = np.float32(O.amax(view)) if view.size else np.float32(0)
    p0 = {"below": a * np.float32(0.5), "above": a * np.float32(2) + np.float32(1),
          "zero": np.float32(0)}[prior]
    out = Guarded((1,), torch.float32)
    out.t.fill_(float(p0))
    d = dev_bf16(big) if big.size else torch.empty((rows, ld), dtype=torch.bfloat16, device="cuda")
    L.fp8_amax_acc(d[:, :cols], out.t)
    torch.cuda.synchronize()
    out.check()
    assert bits(out.np())[0] == bits(max(a, p0))


@pytest.mark.parametrize("shape,ld,c0", [((64, 300), 512, 8), ((33, 77), 101, 0), ((1000, 8), 16, 0),
                                         ((5, 4096), 4104, 8), ((2, 1), 9, 0), ((3, 5), 11, 0)])
def test_amax_strided_rows(O, L, shape, ld, c0):
    """A [rows][cols] view of a wider buffer (row stride ld): 16-byte row
    loads when ld % 8 == 0, element loads otherwise."""
    rows, cols = shape
    rng = np.random.default_rng(rows + ld)
    big = datagen.normal(rng, (rows, ld), 1.0)
    big[:, :c0] = datagen.bf16_bits(np.full((rows, c0), 1e4, np.float32))   # outside the view
    big[:, c0 + cols:] = datagen.bf16_bits(np.full((rows, ld - c0 - cols), -2e4, np.float32))
    view = np.ascontiguousarray(big[:, c0:c0 + cols])
    view.reshape(-1)[rows * cols // 2] = datagen.bf16_bits(np.array([-77.0], np.float32))[0]
    big[:, c0:c0 + cols] = view
    d = dev_bf16(big)
    x = d[:, c0:c0 + cols]
    out = Guarded((1,), torch.float32)
    L.fp8_amax(x, out.t)
    torch.cuda.synchronize()
    out.check()
    assert bits(out.np())[0] == bits(O.amax(view))


# ----------------------------------------------------------------- scale ---
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("margin", [0, 3])
def test_compute_scale(O, L, fmt, margin):
    say("compute_scale", fmt, margin)
    rng = np.random.default_rng(5 + fmt)
    a = np.exp2(rng.uniform(-140, 128, 4096)).astype(np.float32)
    a[:16] = [0, np.inf, np.nan, 1e-45, 1e-40, 448, 57344, 3.4e38, 1, 2 ** -126, 2 ** -130,
              0.1, 7, 1e-38, 1e30, 5e-39]
    sc = torch.empty(a.size, dtype=torch.float32, device="cuda")
    si = torch.empty_like(sc)
    L.fp8_compute_scale(dev(a), fmt, margin, sc, si)
    torch.cuda.synchronize()
    want = [O.compute_scale(v, fmt, margin, 1.0) for v in a]
    assert np.array_equal(bits(sc.cpu().numpy()), bits([w[0] for w in want]))
    assert np.array_equal(bits(si.cpu().numpy()), bits([w[1] for w in want]))


@pytest.mark.parametrize("ln,algo", [(16, 0), (32, 0), (16, 1), (1, 0), (63, 0), (64, 0), (65, 0),
                                     (130, 0), (1024, 0), (1024, 1)])
def test_history_update(O, L, ln, algo):
    say("history", ln, algo)
    rng = np.random.default_rng(ln + algo)
    n, steps = 5, 50
    fmts = [0, 0, 1]
    am = np.abs(rng.standard_normal((steps, n))).astype(np.float32) * np.float32(10)
    am[3, 0] = 1000.0            # spike
    am[:4, 1] = 0.0              # all-zero tensor for the first steps
    am[7, 2] = np.nan
    am[9, 3] = np.inf
    am[11:, 4] = 2.0 ** -140     # subnormal amax: the scale clamps to FLT_MAX
    for fmt in fmts[:2]:
        h = np.zeros((n, ln), np.float32); s = np.ones(n, np.float32); si = np.ones(n, np.float32)
        if ln > 32:   # a full window: every entry, chunk boundaries included, holds a value
            h = (np.abs(rng.standard_normal((n, ln))) * 3).astype(np.float32)
            h[2, ln - 2] = 500.0   # about to leave the window after one step
        hd, sd, sid = dev(h), dev(s), dev(si)
        for t in range(steps):
            L.fp8_amax_history_update(hd, dev(am[t]), fmt, 0, algo, sd, sid)
            O.history_update(h, am[t], fmt, 0, algo, s, si)
            torch.cuda.synchronize()
            assert np.array_equal(bits(hd.cpu().numpy()), bits(h)), t
            assert np.array_equal(bits(sd.cpu().numpy()), bits(s)), t
            assert np.array_equal(bits(sid.cpu().numpy()), bits(si)), t


# ------------------------------------------------------------------ cast ---
def _scales(fmt):
    rng = np.random.default_rng(17 + fmt)
    s = [1.0, 2.0 ** -20, 2.0 ** 20, 3.0, 0.7, 1.0 + 2.0 ** -23, 3.4e38, 1e-30]
    s += list((np.float32(448.0 if fmt == 0 else 57344.0)
               / np.exp2(rng.uniform(-12, 12, 8))).astype(np.float32))
    return [np.float32(v) for v in s]


@pytest.mark.parametrize("fmt", [0, 1])
def test_cast_all_bf16_patterns(O, L, fmt):
    """Every bf16 pattern (NaN, Inf, subnormals, signed zeros included) times
    a set of scales, through the flat, transposed and amax-fused kernels."""
    cast = L.fp8_cast_e4m3 if fmt == 0 else L.fp8_cast_e5m2
    xd = dev_bf16(ALL_BF16)
    for s in _scales(fmt):
        say("cast all-bf16", fmt, float(s))
        want = O.cast(ALL_BF16, s, fmt)
        sdev = dev(np.array([s], np.float32))
        y = Guarded((256, 256), torch.uint8)
        cast(xd, sdev, y=y.t)
        y2 = Guarded((256, 256), torch.uint8)
        yt = Guarded((256, 256), torch.uint8)
        am = Guarded((1,), torch.float32)
        cast(xd, sdev, y=y2.t, y_t=yt.t, amax_out=am.t)
        torch.cuda.synchronize()
        for g in (y, y2, yt, am):
            g.check()
        got = y.np()
        bad = np.argwhere(got != want)
        assert bad.size == 0, (f"{len(bad)} mismatches, first x=0x{ALL_BF16[tuple(bad[0])]:04x} "
                               f"got 0x{got[tuple(bad[0])]:02x} want 0x{want[tuple(bad[0])]:02x}")
        assert np.array_equal(y2.np(), want)
        assert np.array_equal(yt.np(), want.T)
        assert bits(am.np())[0] == bits(O.amax(ALL_BF16))


@pytest.mark.parametrize("shape", [(1, 1), (3, 5), (17, 33), (130, 250), (144, 272), (16, 16),
                                   (272, 16), (0, 7), (4096, 4096)])
@pytest.mark.parametrize("fmt", [0, 1])
def test_cast_shapes(O, L, shape, fmt):
    say("cast shape", shape, fmt)
    rng = np.random.default_rng(shape[0] * 7 + shape[1] + fmt)
    x = datagen.normal(rng, shape, 1.0 if fmt == 0 else 1e-4)
    s = np.float32(448.0 if fmt == 0 else 57344.0) / max(O.amax(x), np.float32(1e-30)) * np.float32(1.5)
    cast = L.fp8_cast_e4m3 if fmt == 0 else L.fp8_cast_e5m2
    y = Guarded(shape, torch.uint8)
    yt = Guarded(shape[::-1], torch.uint8)
    am = Guarded((1,), torch.float32)
    cast(dev_bf16(x), dev(np.array([s], np.float32)), y=y.t, y_t=yt.t, amax_out=am.t)
    y1 = Guarded(shape, torch.uint8)
    cast(dev_bf16(x), dev(np.array([s], np.float32)), y=y1.t)
    yt1 = Guarded(shape[::-1], torch.uint8)
    cast(dev_bf16(x), dev(np.array([s], np.float32)), y_t=yt1.t)
    torch.cuda.synchronize()
    for g in (y, yt, am, y1, yt1):
        g.check()
    want = O.cast(x, s, fmt)
    assert np.array_equal(y.np(), want)
    assert np.array_equal(y1.np(), want)
    assert np.array_equal(yt.np(), want.T)
    assert np.array_equal(yt1.np(), want.T)
    assert bits(am.np())[0] == bits(O.amax(x))


# ----------------------------------------- accumulating cast, resetting update ---
@pytest.mark.parametrize("shape", [(3, 5), (17, 33), (144, 272), (272, 16), (1024, 2048)])
@pytest.mark.parametrize("fmt", [0, 1])
def test_cast_amax_acc(O, L, shape, fmt):
    """fp8_cast_amax_acc writes the codes of fp8_cast_e4m3 / e5m2 (flat,
    transposed and both, every kernel path) and leaves
    max(previous slot, amax(x)) in the slot: from 0, from a larger value
    (unchanged), from a smaller one; two tensors into one slot give the
    larger of their amaxes."""
    say("cast amax acc", shape, fmt)
    rng = np.random.default_rng(shape[0] + 3 * shape[1] + fmt)
    x = datagen.normal(rng, shape, 1.0 if fmt == 0 else 1e-4)
    x2 = datagen.normal(rng, shape, 3.0 if fmt == 0 else 3e-4)
    a1, a2 = O.amax(x), O.amax(x2)
    s = np.float32(448.0 if fmt == 0 else 57344.0) / a1
    want = O.cast(x, s, fmt)
    xd, sd = dev_bf16(x), dev(np.array([s], np.float32))
    for start in (0.0, float(a1) * 4.0, float(a1) / 4.0):
        for outs in ("y", "y_t", "both"):
            y = Guarded(shape, torch.uint8) if outs != "y_t" else None
            yt = Guarded(shape[::-1], torch.uint8) if outs != "y" else None
            slot = Guarded((1,), torch.float32)
            slot.t.fill_(start)
            L.fp8_cast_amax_acc(xd, fmt, sd, slot.t, y=y.t if y else None, y_t=yt.t if yt else None)
            torch.cuda.synchronize()
            for g in (y, yt, slot):
                if g is not None:
                    g.check()
            if y is not None:
                assert np.array_equal(y.np(), want), (start, outs)
            if yt is not None:
                assert np.array_equal(yt.np(), want.T), (start, outs)
            assert bits(slot.np())[0] == bits(max(np.float32(start), a1)), (start, outs)
    slot = torch.zeros(1, dtype=torch.float32, device="cuda")
    y = torch.empty(shape, dtype=torch.uint8, device="cuda")
    L.fp8_cast_amax_acc(xd, fmt, sd, slot, y=y)
    L.fp8_cast_amax_acc(dev_bf16(x2), fmt, sd, slot, y=y)
    torch.cuda.synchronize()
    assert bits(slot.cpu().numpy())[0] == bits(max(a1, a2))


@pytest.mark.parametrize("ln,algo", [(16, 0), (16, 1), (65, 0)])
def test_history_update_reset(O, L, ln, algo):
    """The resetting update gives the histories and scales of the plain one,
    step after step, and leaves every consumed amax at 0."""
    say("history reset", ln, algo)
    rng = np.random.default_rng(100 + ln + algo)
    n, steps = 5, 30
    am = np.abs(rng.standard_normal((steps, n))).astype(np.float32) * np.float32(10)
    am[3, 0] = 1000.0
    am[:4, 1] = 0.0
    am[7, 2] = np.nan
    for fmt in (0, 1):
        h = np.zeros((n, ln), np.float32); s = np.ones(n, np.float32); si = np.ones(n, np.float32)
        hd, sd, sid = dev(h), dev(s), dev(si)
        for t in range(steps):
            ad = dev(am[t])
            L.fp8_amax_history_update_reset(hd, ad, fmt, 0, algo, sd, sid)
            O.history_update(h, am[t], fmt, 0, algo, s, si)
            torch.cuda.synchronize()
            assert np.array_equal(bits(hd.cpu().numpy()), bits(h)), t
            assert np.array_equal(bits(sd.cpu().numpy()), bits(s)), t
            assert np.array_equal(bits(sid.cpu().numpy()), bits(si)), t
            assert np.all(bits(ad.cpu().numpy()) == 0), t
