"""Thin Python binding of libfp8lin (the C ABI in include/fp8lin.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Tensors are torch tensors on the GPU (PyTorch provides device
memory and streams); each call passes their device pointers and sizes to the
C function of the same name and raises Fp8Error on a non-OK status.  There
is no fallback: if libfp8lin.so is missing or fails to load, importing this
module raises.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8lin.so")

E4M3, E5M2 = 0, 1
SCALE_TENSOR, SCALE_1x128, SCALE_128x128 = 0, 1, 2
SCALE_1x128_POW2, SCALE_128x128_POW2 = 3, 4
SCALE_ROW = 5
OUT_BF16, OUT_F32, OUT_E4M3, OUT_E5M2 = 0, 1, 2, 3
AMAX_MAX, AMAX_MOST_RECENT = 0, 1

STATUS = {0: "FP8_OK", 1: "FP8_ERR_NULL", 2: "FP8_ERR_SHAPE", 3: "FP8_ERR_ALIGN",
          4: "FP8_ERR_UNSUPPORTED", 5: "FP8_ERR_LAUNCH", 6: "FP8_ERR_ARG"}


class Fp8Error(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({text})")
        self.status = status


class GemmArgs(C.Structure):
    _fields_ = [("M", C.c_int64), ("N", C.c_int64), ("K", C.c_int64),
                ("lda", C.c_int64), ("ldb", C.c_int64), ("ldd", C.c_int64),
                ("A", C.c_void_p), ("a_fmt", C.c_int), ("a_scaling", C.c_int),
                ("a_scale_inv", C.c_void_p),
                ("B", C.c_void_p), ("b_fmt", C.c_int), ("b_scaling", C.c_int),
                ("b_scale_inv", C.c_void_p),
                ("D", C.c_void_p), ("d_dtype", C.c_int), ("d_amax", C.c_void_p),
                ("accumulate", C.c_int),
                ("d_scale", C.c_void_p), ("D_t", C.c_void_p), ("ldt", C.c_int64),
                ("amax_accumulate", C.c_int)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m fp8_mixed_precision_linear_amd.build`")
    L = C.CDLL(LIB_PATH)
    vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int
    sig = {
        "fp8_abi_version": (i32, []),
        "fp8_status_string": (C.c_char_p, [i32]),
        "fp8_amax": (i32, [vp, i64, i64, i64, vp, vp]),
        "fp8_amax_acc": (i32, [vp, i64, i64, i64, vp, vp]),
        "fp8_cast_stats": (i32, [vp, i64, i64, i32, vp, vp, vp]),
        "fp8_compute_scale": (i32, [vp, i64, i32, i32, vp, vp, vp]),
        "fp8_compute_scale_pow2": (i32, [vp, i64, i32, i32, vp, vp, vp]),
        "fp8_amax_history_update": (i32, [vp, i64, i64, vp, i32, i32, i32, vp, vp, vp]),
        "fp8_amax_history_update_pow2": (i32, [vp, i64, i64, vp, i32, i32, i32, vp, vp, vp]),
        "fp8_amax_history_update_reset": (i32, [vp, i64, i64, vp, i32, i32, i32, vp, vp, vp]),
        "fp8_cast_amax_acc": (i32, [vp, i64, i64, i32, vp, vp, vp, vp, vp]),
        "fp8_cast_e4m3": (i32, [vp, i64, i64, vp, vp, vp, vp, vp]),
        "fp8_cast_e5m2": (i32, [vp, i64, i64, vp, vp, vp, vp, vp]),
        "fp8_cast_block": (i32, [vp, i64, i64, i32, i32, vp, vp, vp, vp, vp]),
        "fp8_cast_block_pow2": (i32, [vp, i64, i64, i32, i32, vp, vp, vp, vp, vp]),
        "fp8_cast_rowwise": (i32, [vp, i64, i64, i32, vp, vp, vp, vp, vp]),
        "fp8_cast_sr": (i32, [vp, i64, i64, i32, vp, C.c_uint64, C.c_uint64, vp, vp, vp, vp]),
        "fp8_cast_sr_state": (i32, [vp, i64, i64, i32, vp, vp, C.c_uint64, vp, vp, vp, vp]),
        "fp8_amax_ewma_update": (i32, [vp, i64, vp, C.c_float, i32, i32, vp, vp, vp]),
        "fp8_scaled_gemm": (i32, [C.POINTER(GemmArgs), vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    return L


_L = _load()


def abi_version() -> int:
    return _L.fp8_abi_version()


def status_string(status: int) -> str:
    return _L.fp8_status_string(status).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise Fp8Error(fn, status, status_string(status))


def _ptr(t, dtypes=None, name="tensor"):
    """Device pointer of a GPU tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr() or None


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


_BF16 = (torch.bfloat16,)
_F32 = (torch.float32,)
_I64 = (torch.int64,)
_U8 = (torch.uint8, torch.float8_e4m3fn, torch.float8_e5m2)


def _need(t, n, name):
    """Raise unless tensor t (if given) holds at least n elements: the C ABI
    cannot see buffer sizes, so the binding checks them before any launch."""
    if t is not None and t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements, the call needs {n}")


def _rc(x):
    """(rows, cols) of a tensor viewed as [rows][cols] (1-D: one row)."""
    if x.dim() == 0:
        return 1, 1
    if x.dim() == 1:
        return 1, x.shape[0]
    cols = 1
    for d in x.shape[1:]:
        cols *= d
    return x.shape[0], cols


def _amax(fn, x, amax, stream):
    _need(amax, 1, "amax")
    if x.dim() == 2 and not x.is_contiguous() and x.stride(1) == 1 and x.stride(0) >= x.shape[1]:
        rows, cols, ld = x.shape[0], x.shape[1], x.stride(0)
        if not x.is_cuda or x.dtype not in _BF16:
            raise TypeError("x must be a bf16 GPU tensor")
        xp = x.data_ptr() or None
    else:
        rows, cols = _rc(x)
        ld = cols
        xp = _ptr(x, _BF16, "x")
    _check(fn.__name__, fn(xp, rows, cols, ld, _ptr(amax, _F32, "amax"), _stream(stream)))


def fp8_amax(x, amax, stream=None):
    """amax of x: a contiguous tensor, or a 2-D view whose rows are strided
    (row stride >= number of columns, unit column stride)."""
    _amax(_L.fp8_amax, x, amax, stream)


def fp8_cast_stats(x, fmt, scale, counts, stream=None):
    """Adds the cast's saturated / underflowed element counts of x (scale
    scale[0], format fmt) to counts[0] / counts[1] (an int64 tensor of 2)."""
    rows, cols = _rc(x)
    _need(scale, 1, "scale")
    if counts is None or counts.dtype != torch.int64 or counts.numel() < 2 or not counts.is_cuda:
        raise ValueError("counts must be a GPU int64 tensor of 2")
    _check("fp8_cast_stats",
           _L.fp8_cast_stats(_ptr(x, _BF16, "x"), rows, cols, fmt, _ptr(scale, _F32, "scale"),
                             counts.data_ptr(), _stream(stream)))


def fp8_amax_acc(x, amax_acc, stream=None):
    """fp8_amax max-accumulated into amax_acc (no fill ahead of the kernel)."""
    if amax_acc is None:
        raise ValueError("amax_acc is required")
    _amax(_L.fp8_amax_acc, x, amax_acc, stream)


def _compute_scale(fn, amax, fmt, margin, scale, scale_inv, stream):
    _need(scale, amax.numel(), "scale")
    _need(scale_inv, amax.numel(), "scale_inv")
    _check(fn.__name__,
           fn(_ptr(amax, _F32, "amax"), amax.numel(), fmt, margin,
              _ptr(scale, _F32, "scale"), _ptr(scale_inv, _F32, "scale_inv"), _stream(stream)))


def fp8_compute_scale(amax, fmt, margin, scale, scale_inv, stream=None):
    _compute_scale(_L.fp8_compute_scale, amax, fmt, margin, scale, scale_inv, stream)


def fp8_compute_scale_pow2(amax, fmt, margin, scale, scale_inv, stream=None):
    _compute_scale(_L.fp8_compute_scale_pow2, amax, fmt, margin, scale, scale_inv, stream)


def _history(fn, history, amax_new, fmt, margin, algo, scale, scale_inv, stream):
    n, ln = history.shape
    for name, t in (("amax_new", amax_new), ("scale", scale), ("scale_inv", scale_inv)):
        _need(t, n, name)
    _check(fn.__name__,
           fn(_ptr(history, _F32, "history"), n, ln, _ptr(amax_new, _F32, "amax_new"), fmt, margin,
              algo, _ptr(scale, _F32, "scale"), _ptr(scale_inv, _F32, "scale_inv"), _stream(stream)))


def fp8_amax_history_update(history, amax_new, fmt, margin, algo, scale, scale_inv, stream=None):
    _history(_L.fp8_amax_history_update, history, amax_new, fmt, margin, algo, scale, scale_inv,
             stream)


def fp8_amax_history_update_pow2(history, amax_new, fmt, margin, algo, scale, scale_inv,
                                 stream=None):
    _history(_L.fp8_amax_history_update_pow2, history, amax_new, fmt, margin, algo, scale,
             scale_inv, stream)


def fp8_amax_history_update_reset(history, amax_new, fmt, margin, algo, scale, scale_inv,
                                  stream=None):
    """fp8_amax_history_update, then amax_new is set to 0 (the slots the next
    step's fp8_cast_amax_acc calls accumulate into)."""
    _history(_L.fp8_amax_history_update_reset, history, amax_new, fmt, margin, algo, scale,
             scale_inv, stream)


def fp8_cast_amax_acc(x, fmt, scale, amax_acc, y=None, y_t=None, stream=None):
    """Per-tensor cast with the amax of x max-accumulated into amax_acc."""
    if amax_acc is None:
        raise ValueError("amax_acc is required")
    rows, cols = _cast_sizes(x, scale, y, y_t, amax_acc)
    _check("fp8_cast_amax_acc",
           _L.fp8_cast_amax_acc(_ptr(x, _BF16, "x"), rows, cols, fmt, _ptr(scale, _F32, "scale"),
                                _ptr(y, _U8, "y"), _ptr(y_t, _U8, "y_t"),
                                _ptr(amax_acc, _F32, "amax_acc"), _stream(stream)))


def _cast_sizes(x, scale, y, y_t, amax_out):
    rows, cols = _rc(x)
    _need(scale, 1, "scale")
    _need(y, rows * cols, "y")
    _need(y_t, rows * cols, "y_t")
    _need(amax_out, 1, "amax_out")
    return rows, cols


def _cast(fn, x, scale, y, y_t, amax_out, stream):
    rows, cols = _cast_sizes(x, scale, y, y_t, amax_out)
    _check(fn.__name__, fn(_ptr(x, _BF16, "x"), rows, cols, _ptr(scale, _F32, "scale"),
                           _ptr(y, _U8, "y"), _ptr(y_t, _U8, "y_t"),
                           _ptr(amax_out, _F32, "amax_out"), _stream(stream)))


def fp8_cast_sr(x, fmt, scale, seed, offset=0, y=None, y_t=None, amax_out=None, stream=None):
    rows, cols = _cast_sizes(x, scale, y, y_t, amax_out)
    _check("fp8_cast_sr",
           _L.fp8_cast_sr(_ptr(x, _BF16, "x"), rows, cols, fmt, _ptr(scale, _F32, "scale"),
                          int(seed), int(offset), _ptr(y, _U8, "y"), _ptr(y_t, _U8, "y_t"),
                          _ptr(amax_out, _F32, "amax_out"), _stream(stream)))


def fp8_cast_sr_state(x, fmt, scale, rng_state, advance=1, y=None, y_t=None, amax_out=None,
                      stream=None):
    """Stochastic-rounding cast whose (seed, offset) are read on the device
    from rng_state (an int64 tensor of 2: seed, offset, as unsigned 64-bit
    words); rng_state[1] then moves on by `advance` in stream order, so a
    replayed graph draws fresh words each time."""
    rows, cols = _cast_sizes(x, scale, y, y_t, amax_out)
    if rng_state.numel() < 2:
        raise ValueError("rng_state needs 2 elements (seed, offset)")
    _check("fp8_cast_sr_state",
           _L.fp8_cast_sr_state(_ptr(x, _BF16, "x"), rows, cols, fmt, _ptr(scale, _F32, "scale"),
                                _ptr(rng_state, _I64, "rng_state"), int(advance),
                                _ptr(y, _U8, "y"), _ptr(y_t, _U8, "y_t"),
                                _ptr(amax_out, _F32, "amax_out"), _stream(stream)))


def fp8_amax_ewma_update(ewma, amax_new, beta, fmt, margin, scale, scale_inv, stream=None):
    n = ewma.numel()
    for name, t in (("amax_new", amax_new), ("scale", scale), ("scale_inv", scale_inv)):
        if t.numel() != n:
            raise ValueError(f"{name} must hold {n} floats")
    _check("fp8_amax_ewma_update",
           _L.fp8_amax_ewma_update(_ptr(ewma, _F32, "ewma"), n, _ptr(amax_new, _F32, "amax_new"),
                                   float(beta), fmt, margin, _ptr(scale, _F32, "scale"),
                                   _ptr(scale_inv, _F32, "scale_inv"), _stream(stream)))


def fp8_cast_e4m3(x, scale, y=None, y_t=None, amax_out=None, stream=None):
    _cast(_L.fp8_cast_e4m3, x, scale, y, y_t, amax_out, stream)


def fp8_cast_e5m2(x, scale, y=None, y_t=None, amax_out=None, stream=None):
    _cast(_L.fp8_cast_e5m2, x, scale, y, y_t, amax_out, stream)


def _cast_block(fn, x, fmt, tile, y, scale_inv, y_t, scale_inv_t, stream):
    rows, cols = _rc(x)
    nrb, ncb = (rows + 127) // 128, (cols + 127) // 128
    _need(y, rows * cols, "y")
    _need(y_t, rows * cols, "y_t")
    _need(scale_inv, ncb * (rows if tile == SCALE_1x128 else nrb), "scale_inv")
    _need(scale_inv_t, nrb * (cols if tile == SCALE_1x128 else ncb), "scale_inv_t")
    _check(fn.__name__,
           fn(_ptr(x, _BF16, "x"), rows, cols, fmt, tile, _ptr(y, _U8, "y"),
              _ptr(scale_inv, _F32, "scale_inv"), _ptr(y_t, _U8, "y_t"),
              _ptr(scale_inv_t, _F32, "scale_inv_t"), _stream(stream)))


def fp8_cast_block(x, fmt, tile, y=None, scale_inv=None, y_t=None, scale_inv_t=None, stream=None):
    _cast_block(_L.fp8_cast_block, x, fmt, tile, y, scale_inv, y_t, scale_inv_t, stream)


def fp8_cast_block_pow2(x, fmt, tile, y=None, scale_inv=None, y_t=None, scale_inv_t=None,
                        stream=None):
    _cast_block(_L.fp8_cast_block_pow2, x, fmt, tile, y, scale_inv, y_t, scale_inv_t, stream)


def fp8_cast_rowwise(x, fmt, y=None, scale_inv=None, y_t=None, scale_inv_t=None, stream=None):
    rows, cols = _rc(x)
    _need(y, rows * cols, "y")
    _need(scale_inv, rows, "scale_inv")
    _need(y_t, rows * cols, "y_t")
    _need(scale_inv_t, cols, "scale_inv_t")
    _check("fp8_cast_rowwise",
           _L.fp8_cast_rowwise(_ptr(x, _BF16, "x"), rows, cols, fmt, _ptr(y, _U8, "y"),
                               _ptr(scale_inv, _F32, "scale_inv"), _ptr(y_t, _U8, "y_t"),
                               _ptr(scale_inv_t, _F32, "scale_inv_t"), _stream(stream)))


def fp8_scaled_gemm(A, a_fmt, a_scaling, a_scale_inv, B, b_fmt, b_scaling, b_scale_inv, D,
                    d_amax=None, accumulate=False, stream=None, d_scale=None, d_fmt=None, D_t=None,
                    amax_accumulate=False):
    """D [M][N] = A [M][K] . B [N][K]^T with FP8 codes.  D is a bf16 or fp32
    tensor, or a uint8 tensor of FP8 codes (d_fmt E4M3 / E5M2, quantised
    with d_scale; D_t optional [N][M] transposed codes).  d_amax receives
    max |output|, max-accumulated into its value with amax_accumulate."""
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or tuple(D.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, D {tuple(D.shape)}")
    if D.dtype in _U8:
        if d_fmt not in (E4M3, E5M2):
            raise ValueError("an FP8 output needs d_fmt (E4M3 or E5M2)")
        d_dtype = OUT_E4M3 if d_fmt == E4M3 else OUT_E5M2
        if D_t is not None and tuple(D_t.shape) != (N, M):
            raise ValueError(f"D_t must be [{N}][{M}], got {tuple(D_t.shape)}")
    else:
        d_dtype = {torch.bfloat16: OUT_BF16, torch.float32: OUT_F32}[D.dtype]
    nkb = (K + 127) // 128

    def scales_needed(scaling, rows):
        if scaling in (SCALE_1x128, SCALE_1x128_POW2):
            return nkb * rows
        if scaling in (SCALE_128x128, SCALE_128x128_POW2):
            return nkb * ((rows + 127) // 128)
        return rows if scaling == SCALE_ROW else 1
    if K > 0 and M > 0 and N > 0:
        _need(a_scale_inv, scales_needed(a_scaling, M), "a_scale_inv")
        _need(b_scale_inv, scales_needed(b_scaling, N), "b_scale_inv")
    _need(d_amax, 1, "d_amax")
    _need(d_scale, 1, "d_scale")
    g = GemmArgs(M, N, K, K, K, N,
                 _ptr(A, _U8, "A"), a_fmt, a_scaling, _ptr(a_scale_inv, _F32, "a_scale_inv"),
                 _ptr(B, _U8, "B"), b_fmt, b_scaling, _ptr(b_scale_inv, _F32, "b_scale_inv"),
                 _ptr(D, None, "D"), d_dtype, _ptr(d_amax, _F32, "d_amax"), 1 if accumulate else 0,
                 _ptr(d_scale, _F32, "d_scale"), _ptr(D_t, _U8, "D_t"), M,
                 1 if amax_accumulate else 0)
    _check("fp8_scaled_gemm", _L.fp8_scaled_gemm(C.byref(g), _stream(stream)))
