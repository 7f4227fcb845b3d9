// gemm_big.hip -- the large-tile FP8 GEMM's BF16 / FP32-output kernels and
// the dispatch; the kernel is in gemm_big_kernel.h.
#include "gemm_big_kernel.h"

namespace fp8lin {

bool gemm_big_supported(const GemmParams& p) {
  // buffer offsets are 32-bit: a 256-row panel of each operand must stay
  // below the out-of-range marker; the scale table covers 512 K blocks
  if ((int64_t)BM * p.lda >= (int64_t)kOOB || (int64_t)BN * p.ldb >= (int64_t)kOOB) return false;
  if ((p.M + BM - 1) / BM * ((p.N + BN - 1) / BN) >= (int64_t)1 << 31) return false;
  if ((p.K + BK - 1) / BK > MAX_KB) return false;
  return true;
}

hipError_t launch_gemm_big(const GemmParams& p, hipStream_t s) {
  // per-tensor and per-row scales: the four-wavefront kernel
  const bool per_a = p.a_scaling == 0 || p.a_scaling == 5, per_b = p.b_scaling == 0 || p.b_scaling == 5;
  if (per_a && per_b) return p.d_fp8 ? launch_gemm_w4_fp8out(p, s) : launch_gemm_w4(p, s);
  // power-of-two block scales: the same kernel, scales in the matrix
  // instruction; other block scales: promoted in FP32 by k_gemm_big
  const bool mx = (p.a_scaling == 0 || p.a_scaling >= 3) && (p.b_scaling == 0 || p.b_scaling >= 3);
  if (mx) return p.d_fp8 ? launch_gemm_w4_mx_fp8out(p, s) : launch_gemm_w4_mx(p, s);
  if (p.d_fp8) return launch_gemm_big_fp8out(p, s);
  return launch_gemm_big_out<false>(p, s);
}

}  // namespace fp8lin
