"""GPU parity at the measured workloads' full sizes, in the launch
configuration bench.py times:
  - per-tensor current-scaling forward, X 256x512 (4 outlier columns x50),
    W 512x512;
  - delayed-scaling fwd + dgrad + wgrad at 4096^3 over 16 steps (amax,
    scales and histories bit-exact every step; casts bit-exact; GEMMs on
    sampled rows and columns), and checkpoint / restore of the scale state
    in the middle of the run;
  - block-wise forward at 8192 x 4096 x 14336 and backward (dgrad, wgrad);
  - one transformer-block linear (QKV, 8192 tokens, 8192 -> 10240) in both
    modes.
Casts are compared on every element; GEMMs on 128 sampled rows and 128
sampled columns (seeded), which cover every K block and every N block."""
import numpy as np
import pytest
import torch

from fp8_mixed_precision_linear_amd import datagen
from tests.gpu_util import dev, dev_bf16, gemm_check, say

pytestmark = pytest.mark.gpu

SAMPLE = 128


@pytest.fixture(scope="module")
def L():
    from fp8_mixed_precision_linear_amd import lib
    assert torch.cuda.is_available()
    return lib


def bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def u8(shape):
    return torch.empty(shape, dtype=torch.uint8, device="cuda")


def f32(shape):
    return torch.empty(shape, dtype=torch.float32, device="cuda")


def check_gemm_sampled(O, G_dev, A, af, asc, sa, B, bf, bsc, sb, bf16, seed, a16=None, b16=None,
                       sample=None):
    """Compare GPU output rows/cols (sampled) with the oracle.  A sampled row
    spans every N and K block, a sampled column every M and K block."""
    M, K = A.shape
    N = B.shape[0]
    n_s = SAMPLE if sample is None else sample
    rng = np.random.default_rng(seed)
    ms = np.sort(rng.choice(M, min(n_s, M), replace=False)).astype(np.int64)
    ns = np.sort(rng.choice(N, min(n_s, N), replace=False)).astype(np.int64)
    Gf = G_dev.float()
    rows = Gf[torch.from_numpy(ms).cuda()].cpu().numpy()
    cols = Gf[:, torch.from_numpy(ns).cuda()].cpu().numpy()
    worst = []
    for G, sel in ((rows, dict(ms=ms)), (cols, dict(ns=ns))):
        ref = O.gemm(A, af, asc, sa, B, bf, bsc, sb, want=("E", "F", "D", "H"), **sel)
        ok1, ok2, m1, m2 = gemm_check(G, ref, K, bf16=bf16)
        assert ok1 and ok2, (m1, m2)
        worst.append((m1, m2))
    if a16 is not None:  # the unquantised fp64 reference on a smaller sample
        ms2, ns2 = ms[:min(16, len(ms))], ns[:min(32, len(ns))]
        R, Bd = O.gemm_ref_bound(A, af, asc, sa, B, bf, bsc, sb, a16, b16, ms=ms2, ns=ns2)
        G = Gf[torch.from_numpy(ms2).cuda()][:, torch.from_numpy(ns2).cuda()].cpu().numpy()
        assert np.all(np.abs(G - R) <= Bd + (2.0 ** -8 if bf16 else 0) * np.abs(G))
    return worst


# ---------------------------------------------------------------- config 1 ---
def test_config1_current_scaling_forward(O, L):
    say("config1")
    c = datagen.config1()
    x, w = c["x"], c["w"]
    amax = torch.zeros(2, dtype=torch.float32, device="cuda")
    L.fp8_amax(dev_bf16(x), amax[0:1])
    L.fp8_amax(dev_bf16(w), amax[1:2])
    s, si = f32(2), f32(2)
    L.fp8_compute_scale(amax, 0, 0, s, si)
    xq, wtq = u8(x.shape), u8(w.shape[::-1])
    L.fp8_cast_e4m3(dev_bf16(x), s[0:1], y=xq)
    L.fp8_cast_e4m3(dev_bf16(w), s[1:2], y_t=wtq)
    y = torch.empty((256, 512), dtype=torch.bfloat16, device="cuda")
    d_amax = f32(1)
    L.fp8_scaled_gemm(xq, 0, 0, si[0:1], wtq, 0, 0, si[1:2], y, d_amax=d_amax)
    torch.cuda.synchronize()
    ax, aw = O.amax(x), O.amax(w)
    assert bits(amax.cpu().numpy()).tolist() == bits([ax, aw]).tolist()
    sx, six, _ = O.compute_scale(ax, 0)
    sw, siw, _ = O.compute_scale(aw, 0)
    assert bits(s.cpu().numpy()).tolist() == bits([sx, sw]).tolist()
    assert bits(si.cpu().numpy()).tolist() == bits([six, siw]).tolist()
    xr = O.cast(x, sx, 0)
    wtr = O.cast_transpose(w, sw, 0)[1]
    assert np.array_equal(xq.cpu().numpy(), xr)
    assert np.array_equal(wtq.cpu().numpy(), wtr)
    check_gemm_sampled(O, y, xr, 0, 0, np.array([six]), wtr, 0, 0, np.array([siw]), True, 1,
                       a16=x, b16=np.ascontiguousarray(w.T))
    raw = y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert bits(d_amax.cpu().numpy())[0] == (np.uint32(np.max(raw & 0x7FFF)) << 16)


# ---------------------------------------------------------------- config 2 ---
class DelayedRun:
    """The measured delayed-scaling step, run step by step on the GPU."""

    def __init__(self, L, T=4096, DI=4096, DO=4096, fused=False):
        self.L = L
        # fused: casts accumulate into the amax slots that the resetting
        # history update clears (no zeroing kernel before the casts)
        self.fused = fused
        self.xq, self.xtq = u8((T, DI)), u8((DI, T))
        self.wq, self.wtq = u8((DI, DO)), u8((DO, DI))
        self.dyq, self.dytq = u8((T, DO)), u8((DO, T))
        self.y = torch.empty((T, DO), dtype=torch.bfloat16, device="cuda")
        self.dx = torch.empty((T, DI), dtype=torch.bfloat16, device="cuda")
        self.dw = f32((DI, DO))
        self.hist = torch.zeros((3, 16), dtype=torch.float32, device="cuda")
        self.scale = torch.ones(3, dtype=torch.float32, device="cuda")
        self.sinv = torch.ones(3, dtype=torch.float32, device="cuda")
        self.amax = torch.zeros(3, dtype=torch.float32, device="cuda")

    def step(self, x, w, dy):
        if self.fused:
            return self.step_fused(x, w, dy)
        L, s, si = self.L, self.scale, self.sinv
        L.fp8_cast_e4m3(x, s[0:1], y=self.xq, y_t=self.xtq, amax_out=self.amax[0:1])
        L.fp8_cast_e4m3(w, s[1:2], y=self.wq, y_t=self.wtq, amax_out=self.amax[1:2])
        L.fp8_scaled_gemm(self.xq, 0, 0, si[0:1], self.wtq, 0, 0, si[1:2], self.y)
        L.fp8_cast_e5m2(dy, s[2:3], y=self.dyq, y_t=self.dytq, amax_out=self.amax[2:3])
        L.fp8_scaled_gemm(self.dyq, 1, 0, si[2:3], self.wq, 0, 0, si[1:2], self.dx)
        L.fp8_scaled_gemm(self.xtq, 0, 0, si[0:1], self.dytq, 1, 0, si[2:3], self.dw)
        L.fp8_amax_history_update(self.hist[0:2], self.amax[0:2], 0, 0, 0, s[0:2], si[0:2])
        L.fp8_amax_history_update(self.hist[2:3], self.amax[2:3], 1, 0, 0, s[2:3], si[2:3])

    def step_fused(self, x, w, dy):
        L, s, si, am = self.L, self.scale, self.sinv, self.amax
        L.fp8_cast_amax_acc(x, 0, s[0:1], am[0:1], y=self.xq, y_t=self.xtq)
        L.fp8_cast_amax_acc(w, 0, s[1:2], am[1:2], y=self.wq, y_t=self.wtq)
        L.fp8_scaled_gemm(self.xq, 0, 0, si[0:1], self.wtq, 0, 0, si[1:2], self.y)
        L.fp8_cast_amax_acc(dy, 1, s[2:3], am[2:3], y=self.dyq, y_t=self.dytq)
        L.fp8_scaled_gemm(self.dyq, 1, 0, si[2:3], self.wq, 0, 0, si[1:2], self.dx)
        L.fp8_scaled_gemm(self.xtq, 0, 0, si[0:1], self.dytq, 1, 0, si[2:3], self.dw)
        L.fp8_amax_history_update_reset(self.hist[0:2], am[0:2], 0, 0, 0, s[0:2], si[0:2])
        L.fp8_amax_history_update_reset(self.hist[2:3], am[2:3], 1, 0, 0, s[2:3], si[2:3])

    def state(self):
        return (self.hist.cpu().numpy().copy(), self.scale.cpu().numpy().copy(),
                self.sinv.cpu().numpy().copy())


@pytest.fixture(scope="module")
def c2_data():
    out = []
    for t in range(16):
        d = datagen.config2_step(t)
        out.append(d)
    return out


@pytest.mark.parametrize("fused", [False, True])
def test_config2_delayed_16_steps(O, L, c2_data, fused):
    run = DelayedRun(L, fused=fused)
    h = np.zeros((3, 16), np.float32)
    s = np.ones(3, np.float32)
    si = np.ones(3, np.float32)
    fmts = [0, 0, 1]
    for t, d in enumerate(c2_data):
        say("config2 step", t)
        s_used, si_used = s.copy(), si.copy()
        xd, wd, dyd = dev_bf16(d["x"]), dev_bf16(d["w"]), dev_bf16(d["dy"])
        run.step(xd, wd, dyd)
        torch.cuda.synchronize()
        am = np.array([O.amax_parallel(d["x"]), O.amax_parallel(d["w"]), O.amax_parallel(d["dy"])],
                      np.float32)
        if fused:   # consumed: the amaxes are in the history's newest entries
            assert np.all(bits(run.amax.cpu().numpy()) == 0), t
        else:
            assert np.array_equal(bits(run.amax.cpu().numpy()), bits(am)), t
        for i, f in enumerate(fmts):
            hh, ss, sii = h[i:i + 1].copy(), s[i:i + 1].copy(), si[i:i + 1].copy()
            O.history_update(hh, am[i:i + 1], f, 0, 0, ss, sii)
            h[i], s[i], si[i] = hh[0], ss[0], sii[0]
        gh, gs, gsi = run.state()
        assert np.array_equal(bits(gh), bits(h)) and np.array_equal(bits(gs), bits(s)), t
        assert np.array_equal(bits(gsi), bits(si)), t
        if t in (0, 1, 15):  # casts with the scale in force at this step, every byte
            xr = O.cast(d["x"], s_used[0], 0)
            wr = O.cast(d["w"], s_used[1], 0)
            dr = O.cast(d["dy"], s_used[2], 1)
            assert np.array_equal(run.xq.cpu().numpy(), xr)
            assert np.array_equal(run.xtq.cpu().numpy(), xr.T)
            assert np.array_equal(run.wq.cpu().numpy(), wr)
            assert np.array_equal(run.wtq.cpu().numpy(), wr.T)
            assert np.array_equal(run.dyq.cpu().numpy(), dr)
            assert np.array_equal(run.dytq.cpu().numpy(), dr.T)
            if t in (1, 15):
                sa = lambda i: np.array([si_used[i]], np.float32)
                check_gemm_sampled(O, run.y, xr, 0, 0, sa(0), np.ascontiguousarray(wr.T), 0, 0,
                                   sa(1), True, 100 + t,
                                   a16=d["x"], b16=np.ascontiguousarray(d["w"].T))
                check_gemm_sampled(O, run.dx, dr, 1, 0, sa(2), wr, 0, 0, sa(1), True, 200 + t)
                check_gemm_sampled(O, run.dw, np.ascontiguousarray(xr.T), 0, 0, sa(0),
                                   np.ascontiguousarray(dr.T), 1, 0, sa(2), False, 300 + t)


def test_config2_checkpoint_restore_bitexact(O, L, c2_data):
    """Scale state saved after 8 steps and restored into fresh buffers
    continues bit-exactly (histories, scales and every output byte)."""
    say("config2 checkpoint")
    dd = [(dev_bf16(d["x"]), dev_bf16(d["w"]), dev_bf16(d["dy"])) for d in c2_data]
    a = DelayedRun(L)
    for t in range(8):
        a.step(*dd[t])
    torch.cuda.synchronize()
    ck = [v.clone() for v in (a.hist, a.scale, a.sinv)]
    outs_a = []
    for t in range(8, 16):
        a.step(*dd[t])
        outs_a.append([v.clone() for v in (a.y, a.dx, a.dw, a.xq, a.dyq)])
    b = DelayedRun(L)
    b.hist.copy_(ck[0]); b.scale.copy_(ck[1]); b.sinv.copy_(ck[2])
    for i, t in enumerate(range(8, 16)):
        b.step(*dd[t])
        for va, vb in zip(outs_a[i], (b.y, b.dx, b.dw, b.xq, b.dyq)):
            assert torch.equal(va.view(torch.uint8), vb.view(torch.uint8))
    torch.cuda.synchronize()
    for va, vb in zip((a.hist, a.scale, a.sinv), (b.hist, b.scale, b.sinv)):
        assert torch.equal(va.view(torch.int32), vb.view(torch.int32))


# ----------------------------------------------------------- configs 3, 4 ---
@pytest.fixture(scope="module")
def c34():
    c3 = datagen.config3()
    dy = datagen.config4_dy(c3["rng"])
    return c3["x"], c3["w"], dy


def test_config3_blockwise_forward(O, L, c34):
    x, w, _ = c34
    T, DI = x.shape
    DO = w.shape[1]
    say("config3 casts")
    xq, sx = u8((T, DI)), f32((DI // 128, T))
    wq, sw, wtq, swt = u8((DI, DO)), f32((DO // 128, DI // 128)), u8((DO, DI)), f32((DI // 128, DO // 128))
    L.fp8_cast_block(dev_bf16(x), 0, 1, xq, sx)
    L.fp8_cast_block(dev_bf16(w), 0, 2, wq, sw, wtq, swt)
    y = torch.empty((T, DO), dtype=torch.bfloat16, device="cuda")
    L.fp8_scaled_gemm(xq, 0, 1, sx, wtq, 0, 2, swt, y)
    torch.cuda.synchronize()
    ox = O.cast_block(x, 0, O.S1x128, want_y=True)
    ow = O.cast_block(w, 0, O.S128x128, want_y=True, want_t=True)
    assert np.array_equal(xq.cpu().numpy(), ox["y"])
    assert np.array_equal(bits(sx.cpu().numpy()), bits(ox["sinv"]))
    assert np.array_equal(wq.cpu().numpy(), ow["y"])
    assert np.array_equal(wtq.cpu().numpy(), ow["y_t"])
    assert np.array_equal(bits(sw.cpu().numpy()), bits(ow["sinv"]))
    assert np.array_equal(bits(swt.cpu().numpy()), bits(ow["sinv_t"]))
    say("config3 gemm")
    check_gemm_sampled(O, y, ox["y"], 0, 1, ox["sinv"], ow["y_t"], 0, 2, ow["sinv_t"], True, 3,
                       a16=x, b16=np.ascontiguousarray(w.T))


def test_config4_blockwise_backward(O, L, c34):
    x, w, dy = c34
    T, DI = x.shape
    DO = w.shape[1]
    say("config4 casts")
    dyq, sdy, dytq, sdyt = u8((T, DO)), f32((DO // 128, T)), u8((DO, T)), f32((T // 128, DO))
    L.fp8_cast_block(dev_bf16(dy), 1, 1, dyq, sdy, dytq, sdyt)
    xtq, sxt = u8((DI, T)), f32((T // 128, DI))
    L.fp8_cast_block(dev_bf16(x), 0, 1, None, None, xtq, sxt)
    wq, sw = u8((DI, DO)), f32((DO // 128, DI // 128))
    L.fp8_cast_block(dev_bf16(w), 0, 2, wq, sw)
    dx = torch.empty((T, DI), dtype=torch.bfloat16, device="cuda")
    dw = f32((DI, DO))
    L.fp8_scaled_gemm(dyq, 1, 1, sdy, wq, 0, 2, sw, dx)
    L.fp8_scaled_gemm(xtq, 0, 1, sxt, dytq, 1, 1, sdyt, dw)
    torch.cuda.synchronize()
    od = O.cast_block(dy, 1, O.S1x128, want_y=True, want_t=True)
    assert np.array_equal(dyq.cpu().numpy(), od["y"])
    assert np.array_equal(dytq.cpu().numpy(), od["y_t"])
    assert np.array_equal(bits(sdy.cpu().numpy()), bits(od["sinv"]))
    assert np.array_equal(bits(sdyt.cpu().numpy()), bits(od["sinv_t"]))
    ox = O.cast_block(x, 0, O.S1x128, want_y=False, want_t=True)
    assert np.array_equal(xtq.cpu().numpy(), ox["y_t"])
    assert np.array_equal(bits(sxt.cpu().numpy()), bits(ox["sinv_t"]))
    ow = O.cast_block(w, 0, O.S128x128, want_y=True)
    say("config4 dgrad")
    check_gemm_sampled(O, dx, od["y"], 1, 1, od["sinv"], ow["y"], 0, 2, ow["sinv"], True, 4,
                       a16=dy, b16=w)
    say("config4 wgrad")
    check_gemm_sampled(O, dw, ox["y_t"], 0, 1, ox["sinv_t"], od["y_t"], 1, 1, od["sinv_t"], False, 5,
                       a16=np.ascontiguousarray(x.T), b16=np.ascontiguousarray(dy.T))


# ---------------------------------------------------------------- config 5 ---
@pytest.mark.parametrize("mode", ["delayed", "block"])
def test_config5_qkv_linear(O, L, mode):
    say("config5 qkv", mode)
    d = datagen.config5_linear("qkv")
    x, w, dy = d["x"], d["w"], d["dy"]
    T, DI = x.shape
    DO = w.shape[1]
    xd, wd = dev_bf16(x), dev_bf16(w)
    y = torch.empty((T, DO), dtype=torch.bfloat16, device="cuda")
    if mode == "delayed":
        # one step to fill the histories, then the measured step's forward
        hist = torch.zeros((2, 16), dtype=torch.float32, device="cuda")
        s = torch.ones(2, dtype=torch.float32, device="cuda")
        si = torch.ones(2, dtype=torch.float32, device="cuda")
        am = torch.zeros(2, dtype=torch.float32, device="cuda")
        xq, wtq = u8((T, DI)), u8((DO, DI))
        for _ in range(2):
            L.fp8_cast_e4m3(xd, s[0:1], y=xq, amax_out=am[0:1])
            L.fp8_cast_e4m3(wd, s[1:2], y_t=wtq, amax_out=am[1:2])
            s_used = s.cpu().numpy().copy()
            si_used = si.cpu().numpy().copy()
            L.fp8_scaled_gemm(xq, 0, 0, si[0:1], wtq, 0, 0, si[1:2], y)
            L.fp8_amax_history_update(hist, am, 0, 0, 0, s, si)
        torch.cuda.synchronize()
        xr = O.cast(x, s_used[0], 0)
        wr = O.cast(w, s_used[1], 0)
        assert np.array_equal(xq.cpu().numpy(), xr)
        assert np.array_equal(wtq.cpu().numpy(), wr.T)
        check_gemm_sampled(O, y, xr, 0, 0, si_used[0:1], np.ascontiguousarray(wr.T), 0, 0,
                           si_used[1:2], True, 51)
    else:
        xq, sx = u8((T, DI)), f32((DI // 128, T))
        wtq, swt = u8((DO, DI)), f32((DI // 128, DO // 128))
        wq, sw = u8((DI, DO)), f32((DO // 128, DI // 128))
        L.fp8_cast_block(xd, 0, 1, xq, sx)
        L.fp8_cast_block(wd, 0, 2, wq, sw, wtq, swt)
        L.fp8_scaled_gemm(xq, 0, 1, sx, wtq, 0, 2, swt, y)
        torch.cuda.synchronize()
        ox = O.cast_block(x, 0, O.S1x128, want_y=True)
        ow = O.cast_block(w, 0, O.S128x128, want_y=True, want_t=True)
        assert np.array_equal(xq.cpu().numpy(), ox["y"])
        assert np.array_equal(wtq.cpu().numpy(), ow["y_t"])
        check_gemm_sampled(O, y, ox["y"], 0, 1, ox["sinv"], ow["y_t"], 0, 2, ow["sinv_t"], True, 52)


_C5_CACHE = {}
# tokens for the four linears below: their in / out sizes are the
# configuration's; generating 8192 tokens of the 28672-wide activation
# alone takes over a minute of CPU (the QKV test above runs 8192 tokens)
C5_TOKENS = 2048


def _c5(name):
    if name not in _C5_CACHE:
        _C5_CACHE.clear()   # one linear's tensors at a time (up to ~1 GB of bf16)
        _C5_CACHE[name] = datagen.config5_linear(name, scale_rows=C5_TOKENS)
    return _C5_CACHE[name]


@pytest.mark.parametrize("mode", ["delayed", "block"])
@pytest.mark.parametrize("name", ["o", "gate", "up", "down"])
def test_config5_linear_fwd_bwd(O, L, name, mode):
    """The other linears of the transformer-block set (in / out sizes of the
    configuration, C5_TOKENS tokens), forward and backward: casts bit-exact
    against the oracle (every byte and scale),
    FWD / DGRAD / WGRAD on 8 sampled rows and 8 sampled columns each (every
    M, N and K block), with the delayed-scaling state after one filling step
    or with block scales."""
    say("config5", name, mode)
    d = _c5(name)
    x, w, dy = d["x"], d["w"], d["dy"]
    T, DI = x.shape
    DO = w.shape[1]
    xd, wd, dyd = dev_bf16(x), dev_bf16(w), dev_bf16(dy)
    y = torch.empty((T, DO), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((T, DI), dtype=torch.bfloat16, device="cuda")
    dw = f32((DI, DO))
    xq, xtq, wq, wtq = u8((T, DI)), u8((DI, T)), u8((DI, DO)), u8((DO, DI))
    dyq, dytq = u8((T, DO)), u8((DO, T))
    n = 8
    if mode == "delayed":
        # one step fills the histories; the second step is checked
        hist = torch.zeros((3, 16), dtype=torch.float32, device="cuda")
        s = torch.ones(3, dtype=torch.float32, device="cuda")
        si = torch.ones(3, dtype=torch.float32, device="cuda")
        am = torch.zeros(3, dtype=torch.float32, device="cuda")
        for _ in range(2):
            s_used, si_used = s.cpu().numpy().copy(), si.cpu().numpy().copy()
            L.fp8_cast_amax_acc(xd, 0, s[0:1], am[0:1], y=xq, y_t=xtq)
            L.fp8_cast_amax_acc(wd, 0, s[1:2], am[1:2], y=wq, y_t=wtq)
            L.fp8_scaled_gemm(xq, 0, 0, si[0:1], wtq, 0, 0, si[1:2], y)
            L.fp8_cast_amax_acc(dyd, 1, s[2:3], am[2:3], y=dyq, y_t=dytq)
            L.fp8_scaled_gemm(dyq, 1, 0, si[2:3], wq, 0, 0, si[1:2], dx)
            L.fp8_scaled_gemm(xtq, 0, 0, si[0:1], dytq, 1, 0, si[2:3], dw)
            L.fp8_amax_history_update_reset(hist[0:2], am[0:2], 0, 0, 0, s[0:2], si[0:2])
            L.fp8_amax_history_update_reset(hist[2:3], am[2:3], 1, 0, 0, s[2:3], si[2:3])
        torch.cuda.synchronize()
        xr, wr, dr = O.cast(x, s_used[0], 0), O.cast(w, s_used[1], 0), O.cast(dy, s_used[2], 1)
        for got, want in ((xq, xr), (xtq, xr.T), (wq, wr), (wtq, wr.T), (dyq, dr), (dytq, dr.T)):
            assert np.array_equal(got.cpu().numpy(), want)
        sa = lambda i: np.array([si_used[i]], np.float32)
        say("config5 gemms", name)
        check_gemm_sampled(O, y, xr, 0, 0, sa(0), np.ascontiguousarray(wr.T), 0, 0, sa(1), True,
                           61, sample=n)
        check_gemm_sampled(O, dx, dr, 1, 0, sa(2), wr, 0, 0, sa(1), True, 62, sample=n)
        check_gemm_sampled(O, dw, np.ascontiguousarray(xr.T), 0, 0, sa(0),
                           np.ascontiguousarray(dr.T), 1, 0, sa(2), False, 63, sample=n)
    else:
        sx, sxt = f32((DI // 128, T)), f32((T // 128, DI))
        sw, swt = f32((DO // 128, DI // 128)), f32((DI // 128, DO // 128))
        sd, sdt = f32((DO // 128, T)), f32((T // 128, DO))
        L.fp8_cast_block(xd, 0, 1, xq, sx, xtq, sxt)
        L.fp8_cast_block(wd, 0, 2, wq, sw, wtq, swt)
        L.fp8_scaled_gemm(xq, 0, 1, sx, wtq, 0, 2, swt, y)
        L.fp8_cast_block(dyd, 1, 1, dyq, sd, dytq, sdt)
        L.fp8_scaled_gemm(dyq, 1, 1, sd, wq, 0, 2, sw, dx)
        L.fp8_scaled_gemm(xtq, 0, 1, sxt, dytq, 1, 1, sdt, dw)
        torch.cuda.synchronize()
        ox = O.cast_block(x, 0, O.S1x128, want_y=True, want_t=True)
        ow = O.cast_block(w, 0, O.S128x128, want_y=True, want_t=True)
        od = O.cast_block(dy, 1, O.S1x128, want_y=True, want_t=True)
        for got, want in ((xq, ox["y"]), (xtq, ox["y_t"]), (wq, ow["y"]), (wtq, ow["y_t"]),
                          (dyq, od["y"]), (dytq, od["y_t"])):
            assert np.array_equal(got.cpu().numpy(), want)
        for got, want in ((sx, ox["sinv"]), (sxt, ox["sinv_t"]), (sw, ow["sinv"]),
                          (swt, ow["sinv_t"]), (sd, od["sinv"]), (sdt, od["sinv_t"])):
            assert np.array_equal(bits(got.cpu().numpy()), bits(want))
        say("config5 gemms", name)
        check_gemm_sampled(O, y, ox["y"], 0, 1, ox["sinv"], ow["y_t"], 0, 2, ow["sinv_t"], True, 64,
                           sample=n)
        check_gemm_sampled(O, dx, od["y"], 1, 1, od["sinv"], ow["y"], 0, 2, ow["sinv"], True, 65,
                           sample=n)
        check_gemm_sampled(O, dw, ox["y_t"], 0, 1, ox["sinv_t"], od["y_t"], 1, 1, od["sinv_t"],
                           False, 66, sample=n)
