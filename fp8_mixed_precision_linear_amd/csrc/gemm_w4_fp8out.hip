// gemm_w4_fp8out.hip -- the four-wavefront per-tensor FP8 GEMM's FP8-output
// kernels (their own translation unit, compiled in parallel with the others).
#include "gemm_w4_kernel.h"

namespace fp8lin {

hipError_t launch_gemm_w4_fp8out(const GemmParams& p, hipStream_t s) {
  return launch_w4_out<true, false>(p, s);
}

}  // namespace fp8lin
