// launch.h -- host-side launchers behind the C ABI (internal to the library).
// Each launcher assumes its arguments were validated by the entry point in
// abi.hip and returns the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8lin {

// Compute units of the current device (queried once per device).
int64_t device_cu_count();

// Fill n dwords at p with v (a kernel, so it is safe inside graph capture).
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s);

// amax over n bf16 values (x 16-byte aligned) into *amax: overwritten
// (acc = 0, a fill kernel runs first) or max-accumulated (acc = 1).
hipError_t launch_amax(const uint16_t* x, int64_t n, float* amax, int acc, hipStream_t s);
// the same over [rows][cols] bf16 with row stride ld >= cols (x 16-byte aligned).
hipError_t launch_amax_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float* amax,
                            int acc, hipStream_t s);

// Saturated / underflowed element counts of the per-tensor cast of n bf16
// values (x 16-byte aligned), added to counts[0] / counts[1].
hipError_t launch_cast_stats(const uint16_t* x, int64_t n, const float* scale, int fmt,
                             uint64_t* counts, hipStream_t s);

// pow2 != 0: power-of-two (exponent-bias) scales instead of fmax / amax.
hipError_t launch_compute_scale(const float* amax, int64_t n, int fmt, int margin, int pow2,
                                float* scale, float* scale_inv, hipStream_t s);

// reset != 0: amax_new[i] is set to 0 once consumed.
hipError_t launch_history_update(float* history, int64_t n, int64_t len, float* amax_new,
                                 int fmt, int margin, int algo, int pow2, int reset, float* scale,
                                 float* scale_inv, hipStream_t s);

// Exponentially weighted amax and its scale, n tensors.
hipError_t launch_ewma_update(float* ewma, int64_t n, const float* amax_new, float beta, int fmt,
                              int margin, float* scale, float* scale_inv, hipStream_t s);

// Per-tensor cast with optional transpose and amax (zeroed here first when
// given, unless amax_acc: then max-accumulated into its current value);
// sr != 0: stochastic rounding with Philox words from (seed, offset), or,
// when rng is given, from (rng[0], rng[1]) read on the device, after which
// rng[1] is advanced by `advance`.
hipError_t launch_cast(const uint16_t* x, int64_t rows, int64_t cols, const float* scale, int fmt,
                       uint8_t* y, uint8_t* y_t, float* amax, int amax_acc, int sr, uint64_t seed,
                       uint64_t offset, uint64_t* rng, uint64_t advance, hipStream_t s);

// Block-wise cast (tile: 1 = 1x128, 2 = 128x128; pow2: power-of-two scales).
hipError_t launch_cast_block(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int tile,
                             int pow2, uint8_t* y, float* sinv, uint8_t* y_t, float* sinv_t,
                             hipStream_t s);

// Row-wise cast: per-row scales for y, per-column scales for y_t (either
// output pair may be absent).
hipError_t launch_cast_rowwise(const uint16_t* x, int64_t rows, int64_t cols, int fmt, uint8_t* y,
                               float* sinv, uint8_t* y_t, float* sinv_t, hipStream_t s);

struct GemmParams {
  int64_t M, N, K, lda, ldb, ldd;
  const uint8_t* A;
  int a_fmt, a_scaling;
  const float* a_sinv;
  const uint8_t* B;
  int b_fmt, b_scaling;
  const float* b_sinv;
  void* D;
  int d_f32;
  float* d_amax;  // max |output| is atomically max-ed into it
  int accumulate;
  int amax_acc;             // 0: launch_gemm zeroes *d_amax first; 1: it does not
  int d_fp8;                // 0: BF16/FP32 output; 1: E4M3 codes; 2: E5M2 codes
  const float* d_scale;     // FP8 output: quantisation scale (1 float)
  uint8_t* D_t;             // FP8 output: optional transposed codes [N][ldt]
  int64_t ldt;
};

hipError_t launch_gemm(const GemmParams& p, hipStream_t s);

// Large-tile GEMM (gemm_big.hip): used when supported (32-bit buffer offsets
// cover a 256-row panel of each operand).
bool gemm_big_supported(const GemmParams& p);
hipError_t launch_gemm_big(const GemmParams& p, hipStream_t s);
hipError_t launch_gemm_big_fp8out(const GemmParams& p, hipStream_t s);   // p.d_fp8 != 0
// Per-tensor or per-row scales on both operands: the four-wavefront kernel
// (gemm_w4.hip, gemm_w4_fp8out.hip), under the same size limits.
hipError_t launch_gemm_w4(const GemmParams& p, hipStream_t s);
hipError_t launch_gemm_w4_fp8out(const GemmParams& p, hipStream_t s);   // p.d_fp8 != 0
// Power-of-two block scales (codes 3 / 4, the other operand possibly per
// tensor): the same kernel with the scales in the matrix instruction
// (gemm_w4_mx.hip, gemm_w4_mx_fp8out.hip).
hipError_t launch_gemm_w4_mx(const GemmParams& p, hipStream_t s);
hipError_t launch_gemm_w4_mx_fp8out(const GemmParams& p, hipStream_t s);   // p.d_fp8 != 0

}  // namespace fp8lin
