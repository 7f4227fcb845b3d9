"""The C-ABI library loads and exports every entry point include/fp8lin.h
declares; argument validation rejects bad calls on the host, before any
launch (so these run without a GPU)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8lin.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    from fp8_mixed_precision_linear_amd import lib
    return lib


def test_header_declares_the_layer_calls():
    fns = declared_functions()
    for f in ["fp8_amax", "fp8_compute_scale", "fp8_amax_history_update", "fp8_cast_e4m3",
              "fp8_cast_e5m2", "fp8_cast_block", "fp8_scaled_gemm", "fp8_abi_version",
              "fp8_status_string", "fp8_compute_scale_pow2", "fp8_amax_history_update_pow2",
              "fp8_cast_block_pow2", "fp8_cast_rowwise", "fp8_cast_sr", "fp8_amax_ewma_update",
              "fp8_cast_sr_state", "fp8_amax_acc", "fp8_cast_stats"]:
        assert f in fns


def test_library_exports_every_declared_symbol(L):
    so = C.CDLL(L.LIB_PATH)
    for f in declared_functions():
        assert hasattr(so, f), f"libfp8lin.so does not export {f}"


def test_version_and_status_strings(L):
    assert L.abi_version() == 10
    for s in range(7):
        assert isinstance(L.status_string(s), str) and L.status_string(s)
    assert L.status_string(99) == "unknown status"


def test_host_validation_before_launch(L):
    f = L._L
    # negative sizes
    assert f.fp8_amax(None, -1, 4, 4, None, None) == 2
    assert f.fp8_amax(C.c_void_p(0x1000), 4, 8, 7, C.c_void_p(0x2000), None) == 2   # ld < cols
    # missing output
    assert f.fp8_amax(None, 0, 0, 0, None, None) == 1
    # misaligned input pointer (never dereferenced: rejected first)
    assert f.fp8_amax(C.c_void_p(0x1002), 4, 4, 4, C.c_void_p(0x2000), None) == 3
    assert f.fp8_amax_acc(C.c_void_p(0x1000), 4, 4, 4, None, None) == 1
    assert f.fp8_amax_acc(C.c_void_p(0x1000), 4, 8, 7, C.c_void_p(0x2000), None) == 2
    assert f.fp8_amax_acc(C.c_void_p(0x1002), 4, 4, 4, C.c_void_p(0x2000), None) == 3
    x, s, c = C.c_void_p(0x1000), C.c_void_p(0x2000), C.c_void_p(0x3000)
    assert f.fp8_cast_stats(x, 4, 8, 0, s, None, None) == 1          # counts
    assert f.fp8_cast_stats(None, 4, 8, 0, s, c, None) == 1          # x
    assert f.fp8_cast_stats(x, 4, 8, 0, None, c, None) == 1          # scale
    assert f.fp8_cast_stats(x, -1, 8, 0, s, c, None) == 2
    assert f.fp8_cast_stats(x, 4, 8, 2, s, c, None) == 6
    assert f.fp8_cast_stats(C.c_void_p(0x1008), 4, 8, 0, s, c, None) == 3
    assert f.fp8_cast_stats(x, 4, 8, 0, s, C.c_void_p(0x3004), None) == 3
    assert f.fp8_cast_stats(None, 0, 8, 0, None, c, None) == 0       # empty: nothing to do
    # scale: bad format / margin / n
    assert f.fp8_compute_scale(None, 1, 7, 0, None, None, None) == 6
    assert f.fp8_compute_scale(None, 1, 0, 99, None, None, None) == 6
    assert f.fp8_compute_scale(None, -1, 0, 0, None, None, None) == 2
    assert f.fp8_compute_scale(None, 1, 0, 0, None, None, None) == 1
    assert f.fp8_compute_scale_pow2(None, 1, 7, 0, None, None, None) == 6
    assert f.fp8_compute_scale_pow2(None, 1, 0, 0, None, None, None) == 1
    assert f.fp8_amax_history_update_pow2(None, 1, 0, None, 0, 0, 0, None, None, None) == 2
    assert f.fp8_cast_block_pow2(None, 4, 4, 0, 0, None, None, None, None, None) == 6
    # history: len out of range, bad algo
    assert f.fp8_amax_history_update(None, 1, 0, None, 0, 0, 0, None, None, None) == 2
    assert f.fp8_amax_history_update(None, 1, 16, None, 0, 0, 5, None, None, None) == 6
    # casts: no outputs, misaligned outputs
    assert f.fp8_cast_e4m3(C.c_void_p(0x1000), 4, 4, C.c_void_p(0x2000), None, None, None, None) == 1
    assert f.fp8_cast_e5m2(C.c_void_p(0x1000), 4, 4, C.c_void_p(0x2000), C.c_void_p(0x3001),
                           None, None, None) == 3
    # block cast: bad tile, unpaired scale pointer
    assert f.fp8_cast_block(C.c_void_p(0x1000), 4, 4, 0, 0, C.c_void_p(0x2000),
                            C.c_void_p(0x3000), None, None, None) == 6
    assert f.fp8_cast_block(C.c_void_p(0x1000), 4, 4, 0, 1, C.c_void_p(0x2000), None, None,
                            None, None) == 1
    # row-wise cast: bad format, unpaired or missing outputs, misalignment, sizes
    x, y, s = C.c_void_p(0x1000), C.c_void_p(0x2000), C.c_void_p(0x3000)
    assert f.fp8_cast_rowwise(x, 4, 4, 2, y, s, None, None, None) == 6
    assert f.fp8_cast_rowwise(x, 4, 4, 0, y, None, None, None, None) == 1
    assert f.fp8_cast_rowwise(x, 4, 4, 0, None, None, y, None, None) == 1
    assert f.fp8_cast_rowwise(x, 4, 4, 0, None, None, None, None, None) == 1
    assert f.fp8_cast_rowwise(None, 4, 4, 0, y, s, None, None, None) == 1
    assert f.fp8_cast_rowwise(x, 4, 4, 0, C.c_void_p(0x2008), s, None, None, None) == 3
    assert f.fp8_cast_rowwise(x, 4, 4, 0, y, C.c_void_p(0x3002), None, None, None) == 3
    assert f.fp8_cast_rowwise(x, -1, 4, 0, y, s, None, None, None) == 2
    assert f.fp8_cast_rowwise(None, 0, 4, 0, None, None, None, None, None) == 0   # empty: no-op
    # stochastic-rounding cast: bad format, missing outputs, misalignment
    assert f.fp8_cast_sr(x, 4, 4, 2, s, 1, 0, y, None, None, None) == 6
    assert f.fp8_cast_sr(x, 4, 4, 0, s, 1, 0, None, None, None, None) == 1
    assert f.fp8_cast_sr(x, 4, 4, 1, s, 1, 0, C.c_void_p(0x2004), None, None, None) == 3
    assert f.fp8_cast_sr(x, -4, 4, 1, s, 1, 0, y, None, None, None) == 2
    # the same with device generator state: bad format, missing or misaligned state
    g = C.c_void_p(0x6000)
    assert f.fp8_cast_sr_state(x, 4, 4, 2, s, g, 1, y, None, None, None) == 6
    assert f.fp8_cast_sr_state(x, 4, 4, 1, s, None, 1, y, None, None, None) == 1
    assert f.fp8_cast_sr_state(x, 4, 4, 1, s, C.c_void_p(0x6004), 1, y, None, None, None) == 3
    assert f.fp8_cast_sr_state(x, 4, 4, 1, s, g, 1, None, None, None, None) == 1
    assert f.fp8_cast_sr_state(x, -4, 4, 1, s, g, 1, y, None, None, None) == 2
    a = C.c_void_p(0x5000)
    # accumulating cast: bad format, missing amax slot or outputs, misaligned slot
    assert f.fp8_cast_amax_acc(x, 4, 4, 2, s, y, None, a, None) == 6
    assert f.fp8_cast_amax_acc(x, 4, 4, 0, s, y, None, None, None) == 1
    assert f.fp8_cast_amax_acc(x, 4, 4, 1, s, None, None, a, None) == 1
    assert f.fp8_cast_amax_acc(x, 4, 4, 0, s, y, None, C.c_void_p(0x5002), None) == 3
    assert f.fp8_cast_amax_acc(x, -4, 4, 0, s, y, None, a, None) == 2
    # resetting history update: as the plain update
    assert f.fp8_amax_history_update_reset(None, 1, 0, None, 0, 0, 0, None, None, None) == 2
    assert f.fp8_amax_history_update_reset(None, 1, 16, None, 0, 0, 5, None, None, None) == 6
    assert f.fp8_amax_history_update_reset(None, 1, 16, None, 0, 0, 0, None, None, None) == 1
    # EWMA update: beta outside [0, 1] or NaN, margin, sizes, pointers
    e, a = C.c_void_p(0x4000), C.c_void_p(0x5000)
    assert f.fp8_amax_ewma_update(e, 1, a, 1.5, 0, 0, s, s, None) == 6
    assert f.fp8_amax_ewma_update(e, 1, a, -0.1, 0, 0, s, s, None) == 6
    assert f.fp8_amax_ewma_update(e, 1, a, float("nan"), 0, 0, s, s, None) == 6
    assert f.fp8_amax_ewma_update(e, 1, a, 0.5, 0, 65, s, s, None) == 6
    assert f.fp8_amax_ewma_update(e, 1, a, 0.5, 2, 0, s, s, None) == 6
    assert f.fp8_amax_ewma_update(e, -1, a, 0.5, 0, 0, s, s, None) == 2
    assert f.fp8_amax_ewma_update(e, 1, None, 0.5, 0, 0, s, s, None) == 1
    assert f.fp8_amax_ewma_update(C.c_void_p(0x4002), 1, a, 0.5, 0, 0, s, s, None) == 3
    assert f.fp8_amax_ewma_update(None, 0, None, 0.5, 0, 0, None, None, None) == 0   # n = 0: no-op


def _gemm(L, **kw):
    g = L.GemmArgs(64, 64, 256, 256, 256, 64, 0x1000, 0, 0, 0x2000, 0x3000, 0, 0, 0x4000,
                   0x5000, 0, None, 0)
    for k, v in kw.items():
        setattr(g, k, v)
    return L._L.fp8_scaled_gemm(C.byref(g), None)


def test_gemm_validation(L):
    assert L._L.fp8_scaled_gemm(None, None) == 1
    assert _gemm(L, K=100) == 2                       # K % 16
    assert _gemm(L, K=272, a_scaling=1) == 2          # block modes need K % 128
    assert _gemm(L, lda=128) == 2                     # lda < K
    assert _gemm(L, lda=264, K=256) == 3              # lda % 16
    assert _gemm(L, A=0x1008) == 3                    # A alignment
    assert _gemm(L, a_fmt=3) == 6
    assert _gemm(L, b_scaling=6) == 6
    # per-row scales: with per-tensor or per-row operands only, K % 16
    assert _gemm(L, a_scaling=5, b_scaling=1) == 4
    assert _gemm(L, a_scaling=4, b_scaling=5) == 4
    assert _gemm(L, K=100, a_scaling=5, b_scaling=5) == 2
    assert _gemm(L, K=272, b_scaling=4) == 2          # power-of-two block modes: K % 128 too
    assert _gemm(L, accumulate=1) == 4                # accumulate needs FP32 output
    assert _gemm(L, D=None) == 1
    assert _gemm(L, ldd=10) == 2
    assert _gemm(L, M=-1) == 2
    # FP8 output: scale required, no accumulation, D_t only with FP8 output
    assert _gemm(L, d_dtype=4) == 6
    assert _gemm(L, d_dtype=2) == 1                   # d_scale missing
    assert _gemm(L, d_dtype=3, d_scale=0x6000, accumulate=1) == 4
    assert _gemm(L, D_t=0x7000, ldt=64) == 6          # D_t with a BF16 output
    assert _gemm(L, d_dtype=2, d_scale=0x6000, D_t=0x7000, ldt=10) == 2
    assert _gemm(L, amax_accumulate=2) == 6
    assert _gemm(L, amax_accumulate=-1) == 6


def test_binding_checks_buffer_sizes(L):
    """The C ABI cannot see buffer sizes: the binding refuses undersized
    tensors before any launch (CPU tensors are never passed on)."""
    import torch
    x = torch.zeros((4, 8), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="y holds 31"):
        L.fp8_cast_e4m3(x, torch.ones(1), y=torch.empty(31, dtype=torch.uint8))
    with pytest.raises(ValueError, match="scale_inv holds 3"):
        L.fp8_cast_rowwise(x, 0, y=torch.empty((4, 8), dtype=torch.uint8), scale_inv=torch.empty(3))
    with pytest.raises(ValueError, match="scale_inv_t holds 1"):
        L.fp8_cast_block(x, 0, 1, y_t=torch.empty((8, 4), dtype=torch.uint8),
                         scale_inv_t=torch.empty(1))
    with pytest.raises(ValueError, match="scale holds 1"):
        L.fp8_amax_history_update(torch.zeros((2, 16)), torch.zeros(2), 0, 0, 0, torch.ones(1),
                                  torch.ones(2))
    A = torch.zeros((256, 384), dtype=torch.uint8)
    B = torch.zeros((128, 384), dtype=torch.uint8)
    D = torch.zeros((256, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="a_scale_inv holds 255"):
        L.fp8_scaled_gemm(A, 0, L.SCALE_ROW, torch.ones(255), B, 0, 0, torch.ones(1), D)
    with pytest.raises(ValueError, match="b_scale_inv holds 2"):
        L.fp8_scaled_gemm(A, 0, 0, torch.ones(1), B, 0, L.SCALE_1x128, torch.ones(2), D)
