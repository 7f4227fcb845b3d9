// gemm_big_fp8out.hip -- the large-tile FP8 GEMM's FP8-output (quantising
// epilogue) kernels; the kernel is in gemm_big_kernel.h.
#include "gemm_big_kernel.h"

namespace fp8lin {

hipError_t launch_gemm_big_fp8out(const GemmParams& p, hipStream_t s) {
  return launch_gemm_big_out<true>(p, s);
}

}  // namespace fp8lin
