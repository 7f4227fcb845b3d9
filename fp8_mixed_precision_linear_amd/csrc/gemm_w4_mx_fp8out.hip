// gemm_w4_mx_fp8out.hip -- the four-wavefront FP8 GEMM with power-of-two
// block scales, FP8 output (its own translation unit, compiled in parallel
// with the others); the kernel is in gemm_w4_kernel.h.
#include "gemm_w4_kernel.h"

namespace fp8lin {

hipError_t launch_gemm_w4_mx_fp8out(const GemmParams& p, hipStream_t s) {
  return launch_w4_out<true, true>(p, s);
}

}  // namespace fp8lin
