// gemm_w4.hip -- the four-wavefront per-tensor FP8 GEMM's BF16 / FP32-output
// kernels; the kernel is in gemm_w4_kernel.h.
#include "gemm_w4_kernel.h"

namespace fp8lin {

hipError_t launch_gemm_w4(const GemmParams& p, hipStream_t s) { return launch_w4_out<false, false>(p, s); }

}  // namespace fp8lin
