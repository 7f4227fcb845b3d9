"""GPU parity at the measured workloads' full sizes, in the launch
configuration bench.py times:
  - per-tensor current-scaling forward, X 256x512 (4 outlier columns x50),
    W 512x512;
  - delayed-scaling fwd + dgrad + wgrad at 4096^3 over 16 steps (amax,
    scales and histories bit-exact every step; casts bit-exact; GEMMs on
    sampled rows and columns), and checkpoint / restore of the scale state
    in the middle of the run;
  - block-wise forward at 8192 x 4096 x 14336 and backward (dgrad, wgrad).
Casts are compared on every element; GEMMs on 128 sampled rows and 128
sampled columns (seeded), which cover every K block and every N block,
under the GEMM gate |G - F| <= 1e-3 max(|F|, D/64) (+ the matrix unit's
in-instruction bound H, zero where it sums exactly) on every sampled
element.  The transformer-block linear set is in test_gpu_c5.py."""
import numpy as np
import pytest
import torch

from fp8_mixed_precision_linear_amd import datagen
from tests.gpu_util import dev, dev_bf16, gate_stats, h_sampler, log_gate, say

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
                       sample=None, label=""):
    """Compare GPU output rows/cols (sampled) with the oracle under the GEMM
    gate on every sampled element:
        |G - F| <= 1e-3 max(|F|, D/64) + H
    (plus half a bf16 ulp of F for BF16 outputs), H the oracle's bound on
    what the matrix unit may drop inside one instruction (zero wherever the
    unit sums exactly: see gate_stats); the plain ratio (without H) is
    logged beside it.  A sampled row spans every N and K block, a sampled
    column every M and K block."""
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
    args = (A, af, asc, sa, B, bf, bsc, sb)
    for G, sel, part in ((rows, dict(ms=ms), "rows"), (cols, dict(ns=ns), "cols")):
        ref = O.gemm(*args, want=("E", "F", "D"), **sel)
        st = gate_stats(G, ref, bf16, h_of=h_sampler(O, *args, **sel))
        log_gate(f"{label} {part} M{M} N{N} K{K}", st)
        assert st["max_rel_hw"] <= 1e-3, st
        worst.append(st)
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
                       a16=x, b16=np.ascontiguousarray(w.T), label="config1 fwd")
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
                                   a16=d["x"], b16=np.ascontiguousarray(d["w"].T),
                                   label=f"config2 step{t} fwd")
                check_gemm_sampled(O, run.dx, dr, 1, 0, sa(2), wr, 0, 0, sa(1), True, 200 + t,
                                   label=f"config2 step{t} dgrad")
                check_gemm_sampled(O, run.dw, np.ascontiguousarray(xr.T), 0, 0, sa(0),
                                   np.ascontiguousarray(dr.T), 1, 0, sa(2), False, 300 + t,
                                   label=f"config2 step{t} wgrad")


@pytest.mark.parametrize("fused", [False, True])
def test_delayed_step_graph_replays_vs_oracle(O, L, c2_data, fused):
    """The delayed-scaling step captured once into a HIP graph and replayed
    on four steps of inputs (copied into the captured input buffers between
    replays, eager work and synchronisation in between): after every replay
    the histories and scales equal the oracle's recurrence bit for bit, every
    cast byte equals the oracle's cast at the scale in force, and the three
    GEMMs pass the gate on sampled rows and columns (steps 1 and 3).
    Operands are the 1024 x 1024 leading blocks of the 4096^3 workload's
    tensors (four 256 x 256 tiles per side)."""
    n = 1024
    run = DelayedRun(L, T=n, DI=n, DO=n, fused=fused)
    data = [{k: np.ascontiguousarray(d[k][:n, :n]) for k in ("x", "w", "dy")} for d in c2_data[:4]]
    xb, wb, dyb = (torch.empty((n, n), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run.step(xb, wb, dyb)
    torch.cuda.synchronize()
    h = np.zeros((3, 16), np.float32)
    s = np.ones(3, np.float32)
    si = np.ones(3, np.float32)
    fmts = [0, 0, 1]
    for t, d in enumerate(data):
        say("graph replay vs oracle", fused, t)
        s_used, si_used = s.copy(), si.copy()
        xb.copy_(dev_bf16(d["x"])); wb.copy_(dev_bf16(d["w"])); dyb.copy_(dev_bf16(d["dy"]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        am = np.array([O.amax(d["x"]), O.amax(d["w"]), O.amax(d["dy"])], np.float32)
        for i, f in enumerate(fmts):
            hh, ss, sii = h[i:i + 1].copy(), s[i:i + 1].copy(), si[i:i + 1].copy()
            O.history_update(hh, am[i:i + 1], f, 0, 0, ss, sii)
            h[i], s[i], si[i] = hh[0], ss[0], sii[0]
        gh, gs, gsi = run.state()
        assert np.array_equal(bits(gh), bits(h)) and np.array_equal(bits(gs), bits(s)), t
        assert np.array_equal(bits(gsi), bits(si)), t
        xr, wr, dr = O.cast(d["x"], s_used[0], 0), O.cast(d["w"], s_used[1], 0), O.cast(d["dy"], s_used[2], 1)
        for got, want in ((run.xq, xr), (run.xtq, xr.T), (run.wq, wr), (run.wtq, wr.T),
                          (run.dyq, dr), (run.dytq, dr.T)):
            assert np.array_equal(got.cpu().numpy(), want), t
        if t in (1, 3):
            sa = lambda i: np.array([si_used[i]], np.float32)
            check_gemm_sampled(O, run.y, xr, 0, 0, sa(0), np.ascontiguousarray(wr.T), 0, 0, sa(1),
                               True, 400 + t, label=f"graph step{t} fwd")
            check_gemm_sampled(O, run.dx, dr, 1, 0, sa(2), wr, 0, 0, sa(1), True, 500 + t,
                               label=f"graph step{t} dgrad")
            check_gemm_sampled(O, run.dw, np.ascontiguousarray(xr.T), 0, 0, sa(0),
                               np.ascontiguousarray(dr.T), 1, 0, sa(2), False, 600 + t,
                               label=f"graph step{t} wgrad")
    del g


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
                       a16=x, b16=np.ascontiguousarray(w.T), label="config3 fwd")


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
                       a16=dy, b16=w, label="config4 dgrad")
    say("config4 wgrad")
    check_gemm_sampled(O, dw, ox["y_t"], 0, 1, ox["sinv_t"], od["y_t"], 1, 1, od["sinv_t"], False, 5,
                       a16=np.ascontiguousarray(x.T), b16=np.ascontiguousarray(dy.T),
                       label="config4 wgrad")
