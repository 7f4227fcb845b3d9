// gemm_w4_mx.hip -- the four-wavefront FP8 GEMM with power-of-two block
// scales applied inside the matrix instruction, BF16 / FP32 output; the
// kernel is in gemm_w4_kernel.h.
#include "gemm_w4_kernel.h"

namespace fp8lin {

hipError_t launch_gemm_w4_mx(const GemmParams& p, hipStream_t s) { return launch_w4_out<false, true>(p, s); }

}  // namespace fp8lin
