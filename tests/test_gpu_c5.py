"""GPU parity on the transformer-block linear set at its full size: hidden
8192, FFN 28672, 8192 tokens; QKV 8192 -> 10240, O 8192 -> 8192, gate and up
8192 -> 28672 each, down 28672 -> 8192; forward, dgrad and wgrad of every
linear, in per-tensor delayed scaling (one step fills the histories, the
second step is checked) and in block-wise scaling (1x128 activation and
gradient tiles, 128x128 weight blocks).

Every cast byte and every scale is compared with the oracle; each GEMM on
64 sampled rows and 64 sampled columns (every M, N and K block) under the
GEMM gate |G - F| <= 1e-3 max(|F|, D/64) (+ the matrix unit's
in-instruction bound, see check_gemm_sampled), and on a 16 x 32 sub-sample
against the fp64 GEMM of the unquantised bf16 data within its a-priori
bound."""
import numpy as np
import pytest
import torch

from fp8_mixed_precision_linear_amd import datagen
from tests.gpu_util import dev_bf16, say
from tests.test_gpu_configs import check_gemm_sampled

pytestmark = pytest.mark.gpu

SAMPLE = 64
CASES = [(n, m) for n in ("qkv", "o", "gate", "up", "down") for m in ("delayed", "block")]


@pytest.fixture(scope="module")
def L():
    from fp8_mixed_precision_linear_amd import lib
    assert torch.cuda.is_available()
    return lib


_CACHE = {}


def _linear(name):
    if name not in _CACHE:
        _CACHE.clear()   # one linear's tensors at a time (up to ~1.4 GB of bf16)
        say("config5 generating", name)
        _CACHE[name] = datagen.config5_linear(name)
    return _CACHE[name]


def bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def u8(shape):
    return torch.empty(shape, dtype=torch.uint8, device="cuda")


def f32(shape):
    return torch.empty(shape, dtype=torch.float32, device="cuda")


def same(got: torch.Tensor, want: np.ndarray) -> bool:
    return np.array_equal(got.cpu().numpy(), want)


@pytest.mark.parametrize("name,mode", CASES)
def test_config5_linear_full_size(O, L, name, mode):
    d = _linear(name)
    x, w, dy = d["x"], d["w"], d["dy"]
    T, DI = x.shape
    DO = w.shape[1]
    say("config5", name, mode, f"T={T} in={DI} out={DO}")
    xd, wd, dyd = dev_bf16(x), dev_bf16(w), dev_bf16(dy)
    y = torch.empty((T, DO), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((T, DI), dtype=torch.bfloat16, device="cuda")
    dw = f32((DI, DO))
    xq, xtq, wq, wtq = u8((T, DI)), u8((DI, T)), u8((DI, DO)), u8((DO, DI))
    dyq, dytq = u8((T, DO)), u8((DO, T))
    x_t, w_t, dy_t = (np.ascontiguousarray(a.T) for a in (x, w, dy))
    lab = f"config5 {name} {mode}"
    if mode == "delayed":
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
        # the step-0 update made the scales those of current scaling
        amx = [O.amax_parallel(a) for a in (x, w, dy)]
        for i, (a, f) in enumerate(zip(amx, (0, 0, 1))):
            sc, sci, _ = O.compute_scale(a, f)
            assert bits(s_used[i]) == bits(sc) and bits(si_used[i]) == bits(sci), (name, i)
        say("config5 casts", name)
        xr, wr, dr = O.cast(x, s_used[0], 0), O.cast(w, s_used[1], 0), O.cast(dy, s_used[2], 1)
        for got, want in ((xq, xr), (xtq, xr.T), (wq, wr), (wtq, wr.T), (dyq, dr), (dytq, dr.T)):
            assert same(got, want)
        sa = lambda i: np.array([si_used[i]], np.float32)
        wtr = np.ascontiguousarray(wr.T)
        say("config5 fwd", name)
        check_gemm_sampled(O, y, xr, 0, 0, sa(0), wtr, 0, 0, sa(1), True, 61, a16=x, b16=w_t,
                           sample=SAMPLE, label=lab + " fwd")
        say("config5 dgrad", name)
        check_gemm_sampled(O, dx, dr, 1, 0, sa(2), wr, 0, 0, sa(1), True, 62, a16=dy, b16=w,
                           sample=SAMPLE, label=lab + " dgrad")
        say("config5 wgrad", name)
        check_gemm_sampled(O, dw, np.ascontiguousarray(xr.T), 0, 0, sa(0),
                           np.ascontiguousarray(dr.T), 1, 0, sa(2), False, 63, a16=x_t, b16=dy_t,
                           sample=SAMPLE, label=lab + " wgrad")
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
        say("config5 casts", name)
        ox = O.cast_block(x, 0, O.S1x128, want_y=True, want_t=True)
        ow = O.cast_block(w, 0, O.S128x128, want_y=True, want_t=True)
        od = O.cast_block(dy, 1, O.S1x128, want_y=True, want_t=True)
        for got, want in ((xq, ox["y"]), (xtq, ox["y_t"]), (wq, ow["y"]), (wtq, ow["y_t"]),
                          (dyq, od["y"]), (dytq, od["y_t"])):
            assert same(got, want)
        for got, want in ((sx, ox["sinv"]), (sxt, ox["sinv_t"]), (sw, ow["sinv"]),
                          (swt, ow["sinv_t"]), (sd, od["sinv"]), (sdt, od["sinv_t"])):
            assert np.array_equal(bits(got.cpu().numpy()), bits(want))
        say("config5 fwd", name)
        check_gemm_sampled(O, y, ox["y"], 0, 1, ox["sinv"], ow["y_t"], 0, 2, ow["sinv_t"], True, 64,
                           a16=x, b16=w_t, sample=SAMPLE, label=lab + " fwd")
        say("config5 dgrad", name)
        check_gemm_sampled(O, dx, od["y"], 1, 1, od["sinv"], ow["y"], 0, 2, ow["sinv"], True, 65,
                           a16=dy, b16=w, sample=SAMPLE, label=lab + " dgrad")
        say("config5 wgrad", name)
        check_gemm_sampled(O, dw, ox["y_t"], 0, 1, ox["sinv_t"], od["y_t"], 1, 1, od["sinv_t"],
                           False, 66, a16=x_t, b16=dy_t, sample=SAMPLE, label=lab + " wgrad")
