// abi.hip -- extern "C" entry points of libfp8lin: host-side argument
// validation, then the launchers.  Nothing is enqueued when validation
// fails; a rejected launch maps to FP8_ERR_LAUNCH.
#include "../../include/fp8lin.h"
#include "launch.h"

using namespace fp8lin;

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline bool fmt_ok(int f) { return f == FP8_E4M3 || f == FP8_E5M2; }
inline bool scaling_ok(int s) {
  return s == FP8_SCALE_TENSOR || s == FP8_SCALE_1x128 || s == FP8_SCALE_128x128 ||
         s == FP8_SCALE_1x128_POW2 || s == FP8_SCALE_128x128_POW2 || s == FP8_SCALE_ROW;
}
inline bool is_block(int s) { return s != FP8_SCALE_TENSOR && s != FP8_SCALE_ROW; }
inline fp8_status launched(hipError_t e) { return e == hipSuccess ? FP8_OK : FP8_ERR_LAUNCH; }

fp8_status cast_common(const void* x, int64_t rows, int64_t cols, const float* scale, uint8_t* y,
                       uint8_t* y_t, float* amax_out, int fmt, int sr, uint64_t seed,
                       uint64_t offset, hipStream_t stream, int amax_acc = 0,
                       uint64_t* rng = nullptr, uint64_t advance = 0) {
  if (rows < 0 || cols < 0) return FP8_ERR_SHAPE;
  const bool empty = rows == 0 || cols == 0;
  if (!empty && (x == nullptr || scale == nullptr || (y == nullptr && y_t == nullptr)))
    return FP8_ERR_NULL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(y_t)) return FP8_ERR_ALIGN;
  if (amax_out && !aligned4(amax_out)) return FP8_ERR_ALIGN;
  return launched(launch_cast(static_cast<const uint16_t*>(x), rows, cols, scale, fmt, y, y_t,
                              amax_out, amax_acc, sr, seed, offset, rng, advance, stream));
}

}  // namespace

extern "C" {

int fp8_abi_version(void) { return FP8LIN_ABI_VERSION; }

const char* fp8_status_string(fp8_status status) {
  switch (status) {
    case FP8_OK: return "ok";
    case FP8_ERR_NULL: return "a required pointer is NULL";
    case FP8_ERR_SHAPE: return "invalid shape";
    case FP8_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case FP8_ERR_UNSUPPORTED: return "unsupported combination";
    case FP8_ERR_LAUNCH: return "kernel launch failed";
    case FP8_ERR_ARG: return "argument out of range";
  }
  return "unknown status";
}

namespace {
fp8_status amax_common(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld, float* amax,
                       int acc, hipStream_t stream) {
  if (rows < 0 || cols < 0 || ld < cols) return FP8_ERR_SHAPE;
  if (amax == nullptr) return FP8_ERR_NULL;
  if (rows > 0 && cols > 0 && x_bf16 == nullptr) return FP8_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned4(amax)) return FP8_ERR_ALIGN;
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  if (ld == cols || rows <= 1) return launched(launch_amax(x, rows * cols, amax, acc, stream));
  return launched(launch_amax_rows(x, rows, cols, ld, amax, acc, stream));
}
}  // namespace

fp8_status fp8_cast_stats(const void* x_bf16, int64_t rows, int64_t cols, fp8_format fmt,
                          const float* scale, uint64_t* counts, hipStream_t stream) {
  if (rows < 0 || cols < 0) return FP8_ERR_SHAPE;
  if (!fmt_ok(fmt)) return FP8_ERR_ARG;
  if (counts == nullptr) return FP8_ERR_NULL;
  if (rows > 0 && cols > 0 && (x_bf16 == nullptr || scale == nullptr)) return FP8_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned4(scale) || (reinterpret_cast<uintptr_t>(counts) & 7u) != 0)
    return FP8_ERR_ALIGN;
  return launched(launch_cast_stats(static_cast<const uint16_t*>(x_bf16), rows * cols, scale, fmt,
                                    counts, stream));
}

fp8_status fp8_amax(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld, float* amax,
                    hipStream_t stream) {
  return amax_common(x_bf16, rows, cols, ld, amax, 0, stream);
}

fp8_status fp8_amax_acc(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld,
                        float* amax_acc, hipStream_t stream) {
  return amax_common(x_bf16, rows, cols, ld, amax_acc, 1, stream);
}

}  // extern "C"

namespace {

fp8_status compute_scale_common(const float* amax, int64_t n, fp8_format fmt, int margin, int pow2,
                                float* scale, float* scale_inv, hipStream_t stream) {
  if (n < 0) return FP8_ERR_SHAPE;
  if (!fmt_ok(fmt) || margin < 0 || margin > 64) return FP8_ERR_ARG;
  if (n > 0 && (amax == nullptr || scale == nullptr || scale_inv == nullptr)) return FP8_ERR_NULL;
  if (!aligned4(amax) || !aligned4(scale) || !aligned4(scale_inv)) return FP8_ERR_ALIGN;
  return launched(launch_compute_scale(amax, n, fmt, margin, pow2, scale, scale_inv, stream));
}

fp8_status history_common(float* history, int64_t n, int64_t len, const float* amax_new,
                          fp8_format fmt, int margin, fp8_amax_algo algo, int pow2, float* scale,
                          float* scale_inv, hipStream_t stream, int reset = 0) {
  if (n < 0 || len < 1 || len > 1024) return FP8_ERR_SHAPE;
  if (!fmt_ok(fmt) || margin < 0 || margin > 64) return FP8_ERR_ARG;
  if (algo != FP8_AMAX_MAX && algo != FP8_AMAX_MOST_RECENT) return FP8_ERR_ARG;
  if (n > 0 && (history == nullptr || amax_new == nullptr || scale == nullptr ||
                scale_inv == nullptr))
    return FP8_ERR_NULL;
  if (!aligned4(history) || !aligned4(amax_new) || !aligned4(scale) || !aligned4(scale_inv))
    return FP8_ERR_ALIGN;
  // amax_new is written only when reset (the entry point that resets takes
  // it as a mutable pointer)
  return launched(launch_history_update(history, n, len, const_cast<float*>(amax_new), fmt, margin,
                                        algo, pow2, reset, scale, scale_inv, stream));
}

fp8_status cast_block_common(const void* x_bf16, int64_t rows, int64_t cols, fp8_format fmt,
                             fp8_scaling tile, int pow2, uint8_t* y, float* scale_inv,
                             uint8_t* y_t, float* scale_inv_t, hipStream_t stream) {
  if (rows < 0 || cols < 0) return FP8_ERR_SHAPE;
  if (!fmt_ok(fmt) || (tile != FP8_SCALE_1x128 && tile != FP8_SCALE_128x128)) return FP8_ERR_ARG;
  if (rows == 0 || cols == 0) return FP8_OK;  // nothing to quantise
  if ((y == nullptr) != (scale_inv == nullptr) || (y_t == nullptr) != (scale_inv_t == nullptr))
    return FP8_ERR_NULL;
  if (y == nullptr && y_t == nullptr) return FP8_ERR_NULL;
  if (x_bf16 == nullptr) return FP8_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(y) || !aligned16(y_t)) return FP8_ERR_ALIGN;
  if (!aligned4(scale_inv) || !aligned4(scale_inv_t)) return FP8_ERR_ALIGN;
  return launched(launch_cast_block(static_cast<const uint16_t*>(x_bf16), rows, cols, fmt, tile,
                                    pow2, y, scale_inv, y_t, scale_inv_t, stream));
}

}  // namespace

extern "C" {

fp8_status fp8_compute_scale(const float* amax, int64_t n, fp8_format fmt, int margin,
                             float* scale, float* scale_inv, hipStream_t stream) {
  return compute_scale_common(amax, n, fmt, margin, 0, scale, scale_inv, stream);
}

fp8_status fp8_compute_scale_pow2(const float* amax, int64_t n, fp8_format fmt, int margin,
                                  float* scale, float* scale_inv, hipStream_t stream) {
  return compute_scale_common(amax, n, fmt, margin, 1, scale, scale_inv, stream);
}

fp8_status fp8_amax_history_update(float* history, int64_t n, int64_t len,
                                   const float* amax_new, fp8_format fmt, int margin,
                                   fp8_amax_algo algo, float* scale, float* scale_inv,
                                   hipStream_t stream) {
  return history_common(history, n, len, amax_new, fmt, margin, algo, 0, scale, scale_inv, stream);
}

fp8_status fp8_amax_history_update_pow2(float* history, int64_t n, int64_t len,
                                        const float* amax_new, fp8_format fmt, int margin,
                                        fp8_amax_algo algo, float* scale, float* scale_inv,
                                        hipStream_t stream) {
  return history_common(history, n, len, amax_new, fmt, margin, algo, 1, scale, scale_inv, stream);
}

fp8_status fp8_amax_history_update_reset(float* history, int64_t n, int64_t len, float* amax_new,
                                         fp8_format fmt, int margin, fp8_amax_algo algo,
                                         float* scale, float* scale_inv, hipStream_t stream) {
  return history_common(history, n, len, amax_new, fmt, margin, algo, 0, scale, scale_inv, stream,
                        1);
}

fp8_status fp8_cast_amax_acc(const void* x_bf16, int64_t rows, int64_t cols, fp8_format fmt,
                             const float* scale, uint8_t* y, uint8_t* y_t, float* amax_acc,
                             hipStream_t stream) {
  if (!fmt_ok(fmt)) return FP8_ERR_ARG;
  if (amax_acc == nullptr) return FP8_ERR_NULL;
  return cast_common(x_bf16, rows, cols, scale, y, y_t, amax_acc, fmt, 0, 0, 0, stream, 1);
}

fp8_status fp8_cast_e4m3(const void* x_bf16, int64_t rows, int64_t cols, const float* scale,
                         uint8_t* y, uint8_t* y_t, float* amax_out, hipStream_t stream) {
  return cast_common(x_bf16, rows, cols, scale, y, y_t, amax_out, FP8_E4M3, 0, 0, 0, stream);
}

fp8_status fp8_cast_e5m2(const void* x_bf16, int64_t rows, int64_t cols, const float* scale,
                         uint8_t* y, uint8_t* y_t, float* amax_out, hipStream_t stream) {
  return cast_common(x_bf16, rows, cols, scale, y, y_t, amax_out, FP8_E5M2, 0, 0, 0, stream);
}

fp8_status fp8_cast_sr(const void* x_bf16, int64_t rows, int64_t cols, fp8_format fmt,
                       const float* scale, uint64_t seed, uint64_t offset, uint8_t* y,
                       uint8_t* y_t, float* amax_out, hipStream_t stream) {
  if (!fmt_ok(fmt)) return FP8_ERR_ARG;
  return cast_common(x_bf16, rows, cols, scale, y, y_t, amax_out, fmt, 1, seed, offset, stream);
}

fp8_status fp8_cast_sr_state(const void* x_bf16, int64_t rows, int64_t cols, fp8_format fmt,
                             const float* scale, uint64_t* rng_state, uint64_t advance,
                             uint8_t* y, uint8_t* y_t, float* amax_out, hipStream_t stream) {
  if (!fmt_ok(fmt)) return FP8_ERR_ARG;
  if (rng_state == nullptr) return FP8_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(rng_state) & 7u) != 0) return FP8_ERR_ALIGN;
  return cast_common(x_bf16, rows, cols, scale, y, y_t, amax_out, fmt, 1, 0, 0, stream, 0,
                     rng_state, advance);
}

fp8_status fp8_amax_ewma_update(float* ewma, int64_t n, const float* amax_new, float beta,
                                fp8_format fmt, int margin, float* scale, float* scale_inv,
                                hipStream_t stream) {
  if (n < 0) return FP8_ERR_SHAPE;
  if (!fmt_ok(fmt) || margin < 0 || margin > 64 || !(beta >= 0.0f && beta <= 1.0f))
    return FP8_ERR_ARG;
  if (n > 0 && (ewma == nullptr || amax_new == nullptr || scale == nullptr ||
                scale_inv == nullptr))
    return FP8_ERR_NULL;
  if (!aligned4(ewma) || !aligned4(amax_new) || !aligned4(scale) || !aligned4(scale_inv))
    return FP8_ERR_ALIGN;
  return launched(launch_ewma_update(ewma, n, amax_new, beta, fmt, margin, scale, scale_inv,
                                     stream));
}

fp8_status fp8_cast_block(const void* x_bf16, int64_t rows, int64_t cols, fp8_format fmt,
                          fp8_scaling tile, uint8_t* y, float* scale_inv, uint8_t* y_t,
                          float* scale_inv_t, hipStream_t stream) {
  return cast_block_common(x_bf16, rows, cols, fmt, tile, 0, y, scale_inv, y_t, scale_inv_t,
                           stream);
}

fp8_status fp8_cast_block_pow2(const void* x_bf16, int64_t rows, int64_t cols, fp8_format fmt,
                               fp8_scaling tile, uint8_t* y, float* scale_inv, uint8_t* y_t,
                               float* scale_inv_t, hipStream_t stream) {
  return cast_block_common(x_bf16, rows, cols, fmt, tile, 1, y, scale_inv, y_t, scale_inv_t,
                           stream);
}

fp8_status fp8_cast_rowwise(const void* x_bf16, int64_t rows, int64_t cols, fp8_format fmt,
                            uint8_t* y, float* scale_inv, uint8_t* y_t, float* scale_inv_t,
                            hipStream_t stream) {
  if (rows < 0 || cols < 0) return FP8_ERR_SHAPE;
  if (!fmt_ok(fmt)) return FP8_ERR_ARG;
  if (rows == 0 || cols == 0) return FP8_OK;  // nothing to quantise
  if ((y == nullptr) != (scale_inv == nullptr) || (y_t == nullptr) != (scale_inv_t == nullptr))
    return FP8_ERR_NULL;
  if (y == nullptr && y_t == nullptr) return FP8_ERR_NULL;
  if (x_bf16 == nullptr) return FP8_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(y) || !aligned16(y_t)) return FP8_ERR_ALIGN;
  if (!aligned4(scale_inv) || !aligned4(scale_inv_t)) return FP8_ERR_ALIGN;
  return launched(launch_cast_rowwise(static_cast<const uint16_t*>(x_bf16), rows, cols, fmt, y,
                                      scale_inv, y_t, scale_inv_t, stream));
}

fp8_status fp8_scaled_gemm(const fp8_gemm_args* a, hipStream_t stream) {
  if (a == nullptr) return FP8_ERR_NULL;
  if (a->M < 0 || a->N < 0 || a->K < 0) return FP8_ERR_SHAPE;
  if (!fmt_ok(a->a_fmt) || !fmt_ok(a->b_fmt)) return FP8_ERR_ARG;
  if (!scaling_ok(a->a_scaling) || !scaling_ok(a->b_scaling)) return FP8_ERR_ARG;
  if (a->d_dtype != FP8_OUT_BF16 && a->d_dtype != FP8_OUT_F32 && a->d_dtype != FP8_OUT_E4M3 &&
      a->d_dtype != FP8_OUT_E5M2)
    return FP8_ERR_ARG;
  const bool fp8_out = a->d_dtype == FP8_OUT_E4M3 || a->d_dtype == FP8_OUT_E5M2;
  if (a->accumulate != 0 && a->accumulate != 1) return FP8_ERR_ARG;
  if (a->amax_accumulate != 0 && a->amax_accumulate != 1) return FP8_ERR_ARG;
  if (a->accumulate && a->d_dtype != FP8_OUT_F32) return FP8_ERR_UNSUPPORTED;
  if (!fp8_out && a->D_t != nullptr) return FP8_ERR_ARG;
  const bool block = is_block(a->a_scaling) || is_block(a->b_scaling);
  // per-row scales are applied after the K sum: not with block operands
  if (block && (a->a_scaling == FP8_SCALE_ROW || a->b_scaling == FP8_SCALE_ROW))
    return FP8_ERR_UNSUPPORTED;
  if (a->K % (block ? 128 : 16) != 0) return FP8_ERR_SHAPE;
  if (a->M > 0 && a->N > 0) {
    if (a->D == nullptr) return FP8_ERR_NULL;
    if (a->ldd < a->N) return FP8_ERR_SHAPE;
    if (a->K > 0) {
      if (a->A == nullptr || a->B == nullptr || a->a_scale_inv == nullptr ||
          a->b_scale_inv == nullptr)
        return FP8_ERR_NULL;
      if (a->lda < a->K || a->ldb < a->K) return FP8_ERR_SHAPE;
      if (a->lda % 16 != 0 || a->ldb % 16 != 0) return FP8_ERR_ALIGN;
      if (!aligned16(a->A) || !aligned16(a->B)) return FP8_ERR_ALIGN;
      if (!aligned4(a->a_scale_inv) || !aligned4(a->b_scale_inv)) return FP8_ERR_ALIGN;
    }
    if (!aligned4(a->D)) return FP8_ERR_ALIGN;
    if (fp8_out) {
      if (a->d_scale == nullptr) return FP8_ERR_NULL;
      if (!aligned4(a->d_scale)) return FP8_ERR_ALIGN;
      if (a->D_t != nullptr && a->ldt < a->M) return FP8_ERR_SHAPE;
    }
  }
  if (a->d_amax && !aligned4(a->d_amax)) return FP8_ERR_ALIGN;
  GemmParams p;
  p.M = a->M; p.N = a->N; p.K = a->K;
  p.lda = a->lda; p.ldb = a->ldb; p.ldd = a->ldd;
  p.A = a->A; p.a_fmt = a->a_fmt; p.a_scaling = a->a_scaling; p.a_sinv = a->a_scale_inv;
  p.B = a->B; p.b_fmt = a->b_fmt; p.b_scaling = a->b_scaling; p.b_sinv = a->b_scale_inv;
  p.D = a->D; p.d_f32 = a->d_dtype == FP8_OUT_F32 ? 1 : 0;
  p.d_amax = a->d_amax; p.accumulate = a->accumulate; p.amax_acc = a->amax_accumulate;
  p.d_fp8 = a->d_dtype == FP8_OUT_E4M3 ? 1 : (a->d_dtype == FP8_OUT_E5M2 ? 2 : 0);
  p.d_scale = fp8_out ? a->d_scale : nullptr;
  p.D_t = fp8_out ? a->D_t : nullptr;
  p.ldt = a->ldt;
  // the quantising epilogue lives in the large-tile kernel only
  if (fp8_out && p.K > 0 && p.M > 0 && p.N > 0 && !gemm_big_supported(p)) return FP8_ERR_UNSUPPORTED;
  return launched(launch_gemm(p, stream));
}

}  // extern "C"
