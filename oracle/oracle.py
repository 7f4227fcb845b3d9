"""ctypes front-end of the plain CPU oracle (fp8_oracle.c, fp8_brute.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library; the only module both sides use is the seeded input
generator (fp8_mixed_precision_linear_amd/datagen.py), which holds no FP8
arithmetic.

Format / scaling / algo codes are the oracle's own: E4M3 = 0, E5M2 = 1;
TENSOR = 0, 1x128 = 1, 128x128 = 2; MAX = 0, MOST_RECENT = 1.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

E4M3, E5M2 = 0, 1
TENSOR, S1x128, S128x128 = 0, 1, 2
ROW = 5
ALGO_MAX, ALGO_MOST_RECENT = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRCS = [os.path.join(_HERE, "fp8_oracle.c"), os.path.join(_HERE, "fp8_brute.c")]
_lib = None


def nthreads() -> int:
    """Worker threads for the oracle: the host's cores, at most 16."""
    return max(1, min(os.cpu_count() or 1, 16))


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no contraction, no fast-math, generic x86-64)."""
    stale = (not os.path.exists(_SO)
             or any(os.path.getmtime(f) > os.path.getmtime(_SO) for f in _SRCS))
    if force or stale:
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fno-strict-aliasing",
               "-Wall", "-pthread", "-shared", "-fPIC", *_SRCS, "-o", _SO + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_SO + ".tmp", _SO)
    return _SO


class _GemmArgs(C.Structure):
    _fields_ = [("M", C.c_int64), ("N", C.c_int64), ("K", C.c_int64),
                ("lda", C.c_int64), ("ldb", C.c_int64),
                ("A", C.c_void_p), ("a_fmt", C.c_int), ("a_scaling", C.c_int), ("a_sinv", C.c_void_p),
                ("B", C.c_void_p), ("b_fmt", C.c_int), ("b_scaling", C.c_int), ("b_sinv", C.c_void_p)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        L = C.CDLL(_SO)
        L.o_bf16_to_f32.restype = C.c_float
        L.o_bf16_to_f32.argtypes = [C.c_uint16]
        L.o_fp8_decode.restype = C.c_double
        L.o_fp8_decode.argtypes = [C.c_uint8, C.c_int]
        L.o_fp8_encode.restype = C.c_uint8
        L.o_fp8_encode.argtypes = [C.c_float, C.c_int]
        L.o_fp8_encode_brute.restype = C.c_uint8
        L.o_fp8_encode_brute.argtypes = [C.c_float, C.c_int]
        L.o_fp8_max.restype = C.c_double
        L.o_fp8_max.argtypes = [C.c_int]
        L.o_amax_bf16.restype = C.c_float
        L.o_amax_bf16.argtypes = [C.c_void_p, C.c_int64]
        L.o_compute_scale.restype = C.c_int
        L.o_compute_scale.argtypes = [C.c_float, C.c_int, C.c_int, C.c_float,
                                      C.POINTER(C.c_float), C.POINTER(C.c_float)]
        L.o_compute_scale_pow2.restype = C.c_int
        L.o_compute_scale_pow2.argtypes = [C.c_float, C.c_int, C.c_int, C.c_float,
                                           C.POINTER(C.c_float), C.POINTER(C.c_float)]
        L.o_pow2_exponent.restype = C.c_int
        L.o_pow2_exponent.argtypes = [C.c_float, C.c_int]
        for nm in ("o_history_update", "o_history_update_pow2"):
            getattr(L, nm).restype = None
            getattr(L, nm).argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_int,
                                       C.c_int, C.c_int, C.c_void_p, C.c_void_p]
        L.o_cast.restype = None
        L.o_cast.argtypes = [C.c_void_p, C.c_int64, C.c_float, C.c_int, C.c_void_p]
        L.o_cast_stats.restype = None
        L.o_cast_stats.argtypes = [C.c_void_p, C.c_int64, C.c_float, C.c_int, C.c_void_p]
        L.o_cast_transpose.restype = None
        L.o_cast_transpose.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_float, C.c_int,
                                       C.c_void_p, C.c_void_p]
        L.o_cast_rowwise.restype = None
        L.o_cast_rowwise.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_int,
                                     C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
        for nm in ("o_cast_block", "o_cast_block_pow2"):
            getattr(L, nm).restype = None
            getattr(L, nm).argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_int, C.c_int,
                                       C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
        L.o_philox4x32_10.restype = None
        L.o_philox4x32_10.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p]
        L.o_sr_word.restype = C.c_uint32
        L.o_sr_word.argtypes = [C.c_uint64, C.c_uint64, C.c_uint64]
        L.o_fp8_encode_sr.restype = C.c_uint8
        L.o_fp8_encode_sr.argtypes = [C.c_float, C.c_int, C.c_uint32]
        L.o_cast_sr.restype = None
        L.o_cast_sr.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_float, C.c_int, C.c_uint64,
                                C.c_uint64, C.c_void_p, C.c_void_p]
        L.o_amax_ewma_update.restype = None
        L.o_amax_ewma_update.argtypes = [C.c_void_p, C.c_int64, C.c_void_p, C.c_float, C.c_int,
                                         C.c_int, C.c_void_p, C.c_void_p]
        L.o_f32_to_bf16.restype = C.c_uint16
        L.o_f32_to_bf16.argtypes = [C.c_float]
        L.o_encode_array.restype = None
        L.o_encode_array.argtypes = [C.c_void_p, C.c_int64, C.c_int, C.c_void_p]
        L.o_decode_array.restype = None
        L.o_decode_array.argtypes = [C.c_void_p, C.c_int64, C.c_int, C.c_void_p]
        L.o_f32_to_bf16_array.restype = None
        L.o_f32_to_bf16_array.argtypes = [C.c_void_p, C.c_int64, C.c_void_p]
        L.o_gemm.restype = None
        L.o_gemm.argtypes = [C.POINTER(_GemmArgs), C.c_void_p, C.c_int64, C.c_void_p, C.c_int64,
                             C.c_void_p, C.c_void_p, C.c_void_p, C.c_int]
        L.o_gemm_h.restype = None
        L.o_gemm_h.argtypes = [C.POINTER(_GemmArgs), C.c_void_p, C.c_int64, C.c_void_p, C.c_int64,
                               C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_int,
                               C.c_int]
        L.o_gemm_ref_bound.restype = None
        L.o_gemm_ref_bound.argtypes = [C.POINTER(_GemmArgs), C.c_void_p, C.c_void_p,
                                       C.c_void_p, C.c_int64, C.c_void_p, C.c_int64,
                                       C.c_void_p, C.c_void_p, C.c_int]
        L.o_encode_exhaustive.restype = C.c_uint64
        L.o_encode_exhaustive.argtypes = [C.c_int, C.c_uint64, C.c_uint64, C.c_int,
                                          C.POINTER(C.c_uint32)]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- codec ---
def fp8_max(fmt: int) -> float:
    return lib().o_fp8_max(fmt)


def decode(codes, fmt: int) -> np.ndarray:
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    lib().o_decode_array(_p(c), c.size, fmt, _p(out))
    return out


def encode(x, fmt: int) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().o_encode_array(_p(x), x.size, fmt, _p(out))
    return out


def encode_brute(x: float, fmt: int) -> int:
    return int(lib().o_fp8_encode_brute(float(np.float32(x)), fmt))


def encode_exhaustive(fmt: int, lo: int = 0, hi: int = 1 << 32, threads: int = None):
    """Bit encoder vs brute-force encoder over binary32 patterns [lo, hi)."""
    bad = C.c_uint32(0)
    n = lib().o_encode_exhaustive(fmt, lo, hi, threads or nthreads(), C.byref(bad))
    return int(n), int(bad.value)


def f32_to_bf16(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().o_f32_to_bf16_array(_p(x), x.size, _p(out))
    return out


# ----------------------------------------------------- amax and scales ---
def amax(x_bf16) -> np.float32:
    x = _c(x_bf16, np.uint16)
    return np.float32(lib().o_amax_bf16(_p(x), x.size))


def amax_parallel(x_bf16) -> np.float32:
    """o_amax over row chunks on worker threads, then the max of the chunk
    maxima (a max is independent of grouping)."""
    x = _c(x_bf16, np.uint16).reshape(-1)
    parts = np.array_split(np.arange(x.size), nthreads()) if x.size else []
    bounds = [(int(p[0]), int(p[-1]) + 1) for p in parts if len(p)]
    L = lib()

    def one(b):
        sub = x[b[0]:b[1]]
        return L.o_amax_bf16(_p(sub), sub.size)

    with ThreadPoolExecutor(len(bounds) or 1) as ex:
        vals = list(ex.map(one, bounds))
    best = np.uint32(0)
    for v in vals:
        b = np.float32(v).view(np.uint32)
        if b > best:
            best = b
    return best.view(np.float32)


def compute_scale(amax_v: float, fmt: int, margin: int = 0, fallback: float = 1.0,
                  pow2: bool = False):
    """(scale, scale_inv, updated).  pow2: the power-of-two (exponent-bias) rule."""
    s, si = C.c_float(), C.c_float()
    fn = lib().o_compute_scale_pow2 if pow2 else lib().o_compute_scale
    ok = fn(float(np.float32(amax_v)), fmt, margin, float(np.float32(fallback)),
            C.byref(s), C.byref(si))
    return np.float32(s.value), np.float32(si.value), bool(ok)


def pow2_exponent(amax_v: float, fmt: int) -> int:
    """Largest e with amax * 2^e <= fmax (before margin and clamping)."""
    return int(lib().o_pow2_exponent(float(np.float32(amax_v)), fmt))


def history_update(history: np.ndarray, amax_new, fmt: int, margin: int, algo: int,
                   scale: np.ndarray, scale_inv: np.ndarray, pow2: bool = False):
    """In-place on history [n][len], scale [n], scale_inv [n] (float32)."""
    assert history.dtype == np.float32 and history.flags.c_contiguous
    assert scale.dtype == np.float32 and scale_inv.dtype == np.float32
    a = _c(amax_new, np.float32)
    n, ln = history.shape
    fn = lib().o_history_update_pow2 if pow2 else lib().o_history_update
    fn(_p(history), n, ln, _p(a), fmt, margin, algo, _p(scale), _p(scale_inv))


def amax_ewma_update(ewma: np.ndarray, amax_new, beta: float, fmt: int, margin: int,
                     scale: np.ndarray, scale_inv: np.ndarray):
    """In-place on ewma [n], scale [n], scale_inv [n] (float32)."""
    for a in (ewma, scale, scale_inv):
        assert a.dtype == np.float32 and a.flags.c_contiguous
    am = _c(amax_new, np.float32)
    lib().o_amax_ewma_update(_p(ewma), ewma.size, _p(am), float(beta), fmt, margin, _p(scale),
                             _p(scale_inv))


# -------------------------------------------------- stochastic rounding ---
def philox4x32_10(ctr, key) -> np.ndarray:
    c = _c(np.asarray(ctr, np.uint32), np.uint32)
    k = _c(np.asarray(key, np.uint32), np.uint32)
    out = np.empty(4, np.uint32)
    lib().o_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def sr_word(seed: int, offset: int, i: int) -> int:
    return int(lib().o_sr_word(seed, offset, i))


def encode_sr(v: float, fmt: int, r: int) -> int:
    return int(lib().o_fp8_encode_sr(float(np.float32(v)), fmt, int(r)))


def cast_sr(x_bf16, s: float, fmt: int, seed: int, offset: int = 0, want_y=True, want_t=False):
    """Per-tensor cast with stochastic rounding; returns (y, y_t) (None where
    not wanted)."""
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    y = np.empty((rows, cols), np.uint8) if want_y else None
    yt = np.empty((cols, rows), np.uint8) if want_t else None
    lib().o_cast_sr(_p(x), rows, cols, float(np.float32(s)), fmt, seed, offset,
                    _p(y) if y is not None else None, _p(yt) if yt is not None else None)
    return y, yt


# -------------------------------------------------------------- casts ---
def cast(x_bf16, s: float, fmt: int) -> np.ndarray:
    x = _c(x_bf16, np.uint16)
    y = np.empty(x.shape, dtype=np.uint8)
    flat_x, flat_y = x.reshape(-1), y.reshape(-1)
    chunks = np.array_split(np.arange(flat_x.size), nthreads()) if flat_x.size else []
    L = lib()

    def one(ch):
        if len(ch) == 0:
            return
        a, b = int(ch[0]), int(ch[-1]) + 1
        L.o_cast(_p(flat_x[a:b]), b - a, float(np.float32(s)), fmt, _p(flat_y[a:b]))

    with ThreadPoolExecutor(max(1, len(chunks))) as ex:
        list(ex.map(one, chunks))
    return y


def cast_stats(x_bf16, s: float, fmt: int) -> tuple:
    """(saturated, underflowed) element counts of the per-tensor cast."""
    x = _c(x_bf16, np.uint16).reshape(-1)
    out = np.zeros(2, np.uint64)
    lib().o_cast_stats(_p(x), x.size, float(np.float32(s)), fmt, _p(out))
    return int(out[0]), int(out[1])


def cast_transpose(x_bf16, s: float, fmt: int):
    """Returns (y [rows][cols], y_t [cols][rows])."""
    y = cast(x_bf16, s, fmt)
    return y, np.ascontiguousarray(y.T)


def cast_transpose_plain(x_bf16, s: float, fmt: int):
    """Single-threaded o_cast_transpose (the plain definition)."""
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    y = np.empty((rows, cols), np.uint8)
    yt = np.empty((cols, rows), np.uint8)
    lib().o_cast_transpose(_p(x), rows, cols, float(np.float32(s)), fmt, _p(y), _p(yt))
    return y, yt


def cast_block(x_bf16, fmt: int, tile: int, want_y=True, want_t=False, plain=False,
               pow2=False):
    """Block-wise cast of x [rows][cols].  Returns dict with y, sinv, y_t,
    sinv_t (the ones requested).  Row chunks of 128*k rows run on worker
    threads (tiles never straddle chunks) unless plain=True.  pow2: the
    tile scales follow the power-of-two (exponent-bias) rule."""
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    nrb, ncb = (rows + 127) // 128, (cols + 127) // 128
    out = {}
    y = np.empty((rows, cols), np.uint8) if want_y else None
    yt = np.empty((cols, rows), np.uint8) if want_t else None
    if tile == S1x128:
        sinv = np.empty((ncb, rows), np.float32) if want_y else None
        sinvt = np.empty((nrb, cols), np.float32) if want_t else None
    else:
        sinv = np.empty((ncb, nrb), np.float32)
        sinvt = np.empty((nrb, ncb), np.float32)
    L = lib()
    nt = 1 if plain else nthreads()
    rb_parts = [p for p in np.array_split(np.arange(nrb), nt) if len(p)]

    def one(part):
        r0, r1 = int(part[0]) * 128, min(rows, (int(part[-1]) + 1) * 128)
        xs = np.ascontiguousarray(x[r0:r1])
        cr = r1 - r0
        ys = np.empty((cr, cols), np.uint8) if y is not None else None
        yts = np.empty((cols, cr), np.uint8) if yt is not None else None
        if tile == S1x128:
            ss = np.empty((ncb, cr), np.float32) if sinv is not None else None
            sts = np.empty(((cr + 127) // 128, cols), np.float32) if sinvt is not None else None
        else:
            ss = np.empty((ncb, (cr + 127) // 128), np.float32)
            sts = np.empty(((cr + 127) // 128, ncb), np.float32)
        (L.o_cast_block_pow2 if pow2 else L.o_cast_block)(_p(xs), cr, cols, fmt, tile,
                       _p(ys) if ys is not None else None, _p(ss) if ss is not None else None,
                       _p(yts) if yts is not None else None, _p(sts) if sts is not None else None)
        rb0, rb1 = r0 // 128, (r1 + 127) // 128
        if ys is not None:
            y[r0:r1] = ys
        if yts is not None:
            yt[:, r0:r1] = yts
        if tile == S1x128:
            if ss is not None:
                sinv[:, r0:r1] = ss
            if sts is not None:
                sinvt[rb0:rb1] = sts
        else:
            sinv[:, rb0:rb1] = ss
            sinvt[rb0:rb1] = sts

    with ThreadPoolExecutor(len(rb_parts) or 1) as ex:
        list(ex.map(one, rb_parts))
    if want_y:
        out["y"], out["sinv"] = y, sinv
    if want_t:
        out["y_t"], out["sinv_t"] = yt, sinvt
    if tile == S128x128:
        out["sinv"], out["sinv_t"] = sinv, sinvt
    return out


def cast_rowwise(x_bf16, fmt: int, want_y=True, want_t=False):
    """Row-wise cast: y with one scale per row, y_t [cols][rows] with one
    scale per column of x.  Returns dict with y, sinv, y_t, sinv_t."""
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    out = {}
    y = np.empty((rows, cols), np.uint8) if want_y else None
    s = np.empty(rows, np.float32) if want_y else None
    yt = np.empty((cols, rows), np.uint8) if want_t else None
    st = np.empty(cols, np.float32) if want_t else None
    lib().o_cast_rowwise(_p(x), rows, cols, fmt, _p(y) if y is not None else None,
                         _p(s) if s is not None else None, _p(yt) if yt is not None else None,
                         _p(st) if st is not None else None)
    if want_y:
        out["y"], out["sinv"] = y, s
    if want_t:
        out["y_t"], out["sinv_t"] = yt, st
    return out


# -------------------------------------------------------------- GEMMs ---
def _gemm_args(A, a_fmt, a_scaling, a_sinv, B, b_fmt, b_scaling, b_sinv, keep):
    A = _c(A, np.uint8)
    B = _c(B, np.uint8)
    a_s = _c(a_sinv, np.float32).reshape(-1)
    b_s = _c(b_sinv, np.float32).reshape(-1)
    keep.extend([A, B, a_s, b_s])
    M, K = A.shape
    N, K2 = B.shape
    assert K == K2
    g = _GemmArgs(M, N, K, K, K, _p(A), a_fmt, a_scaling, _p(a_s), _p(B), b_fmt, b_scaling, _p(b_s))
    return g


def gemm(A, a_fmt, a_scaling, a_sinv, B, b_fmt, b_scaling, b_sinv, ms=None, ns=None,
         want=("E", "F", "D"), hgroup=8, hbits=13):
    """Oracle GEMM D = A B^T (both K-contiguous) with dequant scales.
    Returns dict E (float64), F (float32), D (float64 magnitude), each
    [len(ms)][len(ns)]; with "H" in `want` also the group-truncation bound
    (a tolerance model: groups of `hgroup` consecutive products, products
    below 2^(e_max - hbits) of the group's largest may be lost)."""
    keep = []
    g = _gemm_args(A, a_fmt, a_scaling, a_sinv, B, b_fmt, b_scaling, b_sinv, keep)
    ms = np.arange(g.M, dtype=np.int64) if ms is None else _c(ms, np.int64)
    ns = np.arange(g.N, dtype=np.int64) if ns is None else _c(ns, np.int64)
    E = np.empty((ms.size, ns.size), np.float64) if "E" in want else None
    F = np.empty((ms.size, ns.size), np.float32) if "F" in want else None
    D = np.empty((ms.size, ns.size), np.float64) if "D" in want else None
    H = np.empty((ms.size, ns.size), np.float64) if "H" in want else None
    lib().o_gemm_h(C.byref(g), _p(ms), ms.size, _p(ns), ns.size,
                   _p(E) if E is not None else None, _p(F) if F is not None else None,
                   _p(D) if D is not None else None, _p(H) if H is not None else None,
                   hgroup, hbits, nthreads())
    return {"E": E, "F": F, "D": D, "H": H}


def gemm_ref_bound(A, a_fmt, a_scaling, a_sinv, B, b_fmt, b_scaling, b_sinv,
                   a_bf16, b_bf16, ms=None, ns=None):
    """Unquantised reference R (fp64 GEMM of the bf16 operands a [M][K],
    b [N][K]) and the a-priori bound on |G - R| (without the output
    rounding term)."""
    keep = []
    g = _gemm_args(A, a_fmt, a_scaling, a_sinv, B, b_fmt, b_scaling, b_sinv, keep)
    a16 = _c(a_bf16, np.uint16)
    b16 = _c(b_bf16, np.uint16)
    ms = np.arange(g.M, dtype=np.int64) if ms is None else _c(ms, np.int64)
    ns = np.arange(g.N, dtype=np.int64) if ns is None else _c(ns, np.int64)
    R = np.empty((ms.size, ns.size), np.float64)
    Bd = np.empty((ms.size, ns.size), np.float64)
    lib().o_gemm_ref_bound(C.byref(g), _p(a16), _p(b16), _p(ms), ms.size, _p(ns), ns.size,
                           _p(R), _p(Bd), nthreads())
    return R, Bd
