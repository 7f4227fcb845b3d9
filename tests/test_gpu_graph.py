"""GPU: the delayed-scaling step (three casts with transpose and amax, the
three GEMMs, two amax-history updates) captured into a HIP graph and
replayed gives the eager results bit for bit, replay after replay, with
eager work and synchronisations between the replays.  Every library entry
point the step uses launches kernels only on the caller's stream (zeroing
is done by a fill kernel, not a memset), so the captured sequence is the
eager one.  A GEMM with a fused output amax and a block-wise cast are
captured too."""
import numpy as np
import pytest
import torch

from fp8_mixed_precision_linear_amd import datagen
from tests.gpu_util import dev_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    from fp8_mixed_precision_linear_amd import lib
    assert torch.cuda.is_available()
    return lib


def _capture(fn):
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("fused", [False, True])
def test_delayed_step_graph_replay(L, fused):
    T, DI, DO = 512, 384, 640
    steps = []
    for t in range(2):
        s = datagen.config2_step(t)
        steps.append((dev_bf16(s["x"][:T, :DI]), dev_bf16(s["w"][:DI, :DO]), dev_bf16(s["dy"][:T, :DO])))
    u8 = dict(dtype=torch.uint8, device="cuda")
    out = {
        "xq": torch.empty((T, DI), **u8), "xtq": torch.empty((DI, T), **u8),
        "wq": torch.empty((DI, DO), **u8), "wtq": torch.empty((DO, DI), **u8),
        "dyq": torch.empty((T, DO), **u8), "dytq": torch.empty((DO, T), **u8),
        "y": torch.empty((T, DO), dtype=torch.bfloat16, device="cuda"),
        "dx": torch.empty((T, DI), dtype=torch.bfloat16, device="cuda"),
        "dw": torch.empty((DI, DO), dtype=torch.float32, device="cuda"),
        "hist": torch.zeros((3, 16), dtype=torch.float32, device="cuda"),
        "scale": torch.ones(3, dtype=torch.float32, device="cuda"),
        "sinv": torch.ones(3, dtype=torch.float32, device="cuda"),
        "amax": torch.zeros(3, dtype=torch.float32, device="cuda"),
    }
    o = out

    def step(t):
        x, w, dy = steps[t]
        if fused:   # accumulating casts, resetting history updates
            am = o["amax"]
            L.fp8_cast_amax_acc(x, 0, o["scale"][0:1], am[0:1], y=o["xq"], y_t=o["xtq"])
            L.fp8_cast_amax_acc(w, 0, o["scale"][1:2], am[1:2], y=o["wq"], y_t=o["wtq"])
            L.fp8_scaled_gemm(o["xq"], 0, 0, o["sinv"][0:1], o["wtq"], 0, 0, o["sinv"][1:2], o["y"])
            L.fp8_cast_amax_acc(dy, 1, o["scale"][2:3], am[2:3], y=o["dyq"], y_t=o["dytq"])
            L.fp8_scaled_gemm(o["dyq"], 1, 0, o["sinv"][2:3], o["wq"], 0, 0, o["sinv"][1:2], o["dx"])
            L.fp8_scaled_gemm(o["xtq"], 0, 0, o["sinv"][0:1], o["dytq"], 1, 0, o["sinv"][2:3], o["dw"])
            L.fp8_amax_history_update_reset(o["hist"][0:2], am[0:2], 0, 0, 0, o["scale"][0:2],
                                            o["sinv"][0:2])
            L.fp8_amax_history_update_reset(o["hist"][2:3], am[2:3], 1, 0, 0, o["scale"][2:3],
                                            o["sinv"][2:3])
            return
        L.fp8_cast_e4m3(x, o["scale"][0:1], y=o["xq"], y_t=o["xtq"], amax_out=o["amax"][0:1])
        L.fp8_cast_e4m3(w, o["scale"][1:2], y=o["wq"], y_t=o["wtq"], amax_out=o["amax"][1:2])
        L.fp8_scaled_gemm(o["xq"], 0, 0, o["sinv"][0:1], o["wtq"], 0, 0, o["sinv"][1:2], o["y"])
        L.fp8_cast_e5m2(dy, o["scale"][2:3], y=o["dyq"], y_t=o["dytq"], amax_out=o["amax"][2:3])
        L.fp8_scaled_gemm(o["dyq"], 1, 0, o["sinv"][2:3], o["wq"], 0, 0, o["sinv"][1:2], o["dx"])
        L.fp8_scaled_gemm(o["xtq"], 0, 0, o["sinv"][0:1], o["dytq"], 1, 0, o["sinv"][2:3], o["dw"])
        L.fp8_amax_history_update(o["hist"][0:2], o["amax"][0:2], 0, 0, 0, o["scale"][0:2], o["sinv"][0:2])
        L.fp8_amax_history_update(o["hist"][2:3], o["amax"][2:3], 1, 0, 0, o["scale"][2:3], o["sinv"][2:3])

    def run_two():
        step(0)
        step(1)

    # a non-trivial starting state (a history and scales from one eager step)
    step(1)
    torch.cuda.synchronize()
    # (fused: the amax slots are part of the state, cleared by the update)
    state_keys = ("hist", "scale", "sinv") + (("amax",) if fused else ())
    state0 = {k: o[k].clone() for k in state_keys}
    if fused:
        assert torch.all(state0["amax"] == 0)

    def reset():
        for k, v in state0.items():
            o[k].copy_(v)
        for k in ("xq", "xtq", "wq", "wtq", "dyq", "dytq", "y", "dx", "dw") + (() if fused else ("amax",)):
            o[k].view(torch.uint8).fill_(0x5A)

    reset()
    run_two()
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in o.items()}
    g = _capture(run_two)
    for r in range(3):
        say("graph replay", r)
        reset()
        # unrelated eager work on the stream between replays
        scratch = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in want.items():
            got = o[k]
            assert torch.equal(got.view(torch.uint8), v.view(torch.uint8)), (r, k)
        assert torch.isfinite(scratch)


def test_gemm_amax_and_block_cast_graph_replay(L):
    rng = np.random.default_rng(5)
    M, N, K = 384, 512, 640
    A = torch.from_numpy(rng.integers(0, 0x7E, (M, K), dtype=np.uint8)).cuda()
    B = torch.from_numpy(rng.integers(0, 0x7E, (N, K), dtype=np.uint8)).cuda()
    sa = torch.tensor([0.5], device="cuda")
    sb = torch.tensor([0.25], device="cuda")
    D = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    am = torch.empty(1, dtype=torch.float32, device="cuda")
    x = dev_bf16(datagen.bf16_bits(rng.standard_normal((256, 384)).astype(np.float32)))
    xq, sx = torch.empty((256, 384), dtype=torch.uint8, device="cuda"), torch.empty((3, 256), device="cuda")
    xtq, sxt = torch.empty((384, 256), dtype=torch.uint8, device="cuda"), torch.empty((2, 384), device="cuda")

    def work():
        L.fp8_scaled_gemm(A, 0, 0, sa, B, 0, 0, sb, D, d_amax=am)
        L.fp8_cast_block(x, 0, 1, xq, sx, xtq, sxt)

    outs = (D, am, xq, sx, xtq, sxt)

    def clear():
        for t in outs:
            t.view(torch.uint8).fill_(0xC3)

    clear()
    work()
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]
    g = _capture(work)
    for r in range(3):
        clear()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, w) in enumerate(zip(outs, want)):
            assert torch.equal(t.view(torch.uint8), w.view(torch.uint8)), (r, i)


def test_rowwise_sr_ewma_graph_replay(L):
    """The row-wise cast (four kernels, partial column maxima kept in the
    outputs while it runs), a per-row GEMM with an FP8 output, the
    stochastic-rounding cast and the EWMA update, captured and replayed:
    every replay equals the eager run (the EWMA state is reset first)."""
    rng = np.random.default_rng(9)
    R, Cc, N = 256, 384, 512
    x = dev_bf16(datagen.student_t3(rng, (R, Cc), 1.0))
    w = dev_bf16(datagen.normal(rng, (N, Cc), 0.02))
    u8 = dict(dtype=torch.uint8, device="cuda")
    xq, sx, xtq, sxt = (torch.empty((R, Cc), **u8), torch.empty(R, device="cuda"),
                        torch.empty((Cc, R), **u8), torch.empty(Cc, device="cuda"))
    wq, sw = torch.empty((N, Cc), **u8), torch.empty(N, device="cuda")
    y8, y8t = torch.empty((R, N), **u8), torch.empty((N, R), **u8)
    yam = torch.empty(1, device="cuda")
    so = torch.tensor([3.0], device="cuda")
    sq, sqt, sam = torch.empty((R, Cc), **u8), torch.empty((Cc, R), **u8), torch.empty(1, device="cuda")
    ewma, esc, esi = (torch.zeros(2, device="cuda"), torch.ones(2, device="cuda"),
                      torch.ones(2, device="cuda"))
    am2 = torch.tensor([3.0, 7.0], device="cuda")

    def work():
        L.fp8_cast_rowwise(x, 0, xq, sx, xtq, sxt)
        L.fp8_cast_rowwise(w, 0, wq, sw)
        L.fp8_scaled_gemm(xq, 0, L.SCALE_ROW, sx, wq, 0, L.SCALE_ROW, sw, y8, d_amax=yam,
                          d_scale=so, d_fmt=0, D_t=y8t)
        L.fp8_cast_sr(x, 1, so, 77, 5, y=sq, y_t=sqt, amax_out=sam)
        L.fp8_amax_ewma_update(ewma, am2, 0.5, 0, 0, esc, esi)
        L.fp8_amax_ewma_update(ewma, am2, 0.5, 0, 0, esc, esi)

    outs = (xq, sx, xtq, sxt, wq, sw, y8, y8t, yam, sq, sqt, sam, ewma, esc, esi)

    def clear():
        for t in outs:
            t.view(torch.uint8).fill_(0xC3)
        ewma.zero_()
        esc.fill_(1.0)
        esi.fill_(1.0)

    clear()
    work()
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]
    g = _capture(work)
    for r in range(3):
        say("rowwise/sr/ewma graph replay", r)
        clear()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, wnt) in enumerate(zip(outs, want)):
            assert torch.equal(t.view(torch.uint8), wnt.view(torch.uint8)), (r, i)
