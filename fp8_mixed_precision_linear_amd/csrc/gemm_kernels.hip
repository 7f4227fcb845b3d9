// gemm_kernels.hip -- FP8 scaled GEMM on gfx950 matrix cores (MFMA).
//
// D[m][n] = sum_k A[m][k] B[n][k], A and B FP8 (E4M3 or E5M2, mixed allowed),
// both K-contiguous, FP32 accumulation, dequantisation by inverse scales:
//   tensor x tensor : D = (sum_k a b) * sa * sb, applied in the epilogue;
//   per-row scales  : the same with sa = sa(m), sb = sb(n) ("Per-row vs
//                     per-tensor scaling": one scale per row of an operand
//                     factors out of the sum over k);
//   block modes     : each 128-wide K block is one v_mfma_f32_16x16x128
//                     per 16x16 output tile, accumulated from zero and
//                     promoted into the FP32 accumulator as
//                     acc += P_kb * sa(m,kb) * sb(n,kb).
// [MPG] = "Mixed Precision LLM Training: The Complete Guide":
//   "Transformer Engine internals > Per-tensor scaling" (the matmul result
//   is multiplied by the inverse scales), "Skipping the BAcc accumulator
//   promotion" (FP8 is the multiplicand precision, partial products are
//   accumulated in FP32), "DeepSeek FP8 training recipe in detail >
//   Block-wise scaling at 128 granularity" (block scales applied during the
//   matmul) and "> Mixed-precision accumulation" (FP32 accumulate, BF16 out).
//
// Tiling: a 256-thread workgroup computes a 128x128 output tile; its four
// wavefronts each own 64x64 (4x4 MFMA tiles of 16x16).  The K loop steps
// 128 bytes (one scale block) at a time through double-buffered LDS:
// 128 rows x 128 bytes per operand and stage, each 16-byte chunk stored at
// chunk ^ (row & 7) so that both the 16-byte stores from global memory and
// the 16-byte fragment reads are bank-conflict free.
//
// The MFMA's K order inside one instruction does not matter: lane l feeds
// row (l % 16) of A and row (l % 16) of B with the same 32 bytes of K
// (chunks 2*(l/16) and 2*(l/16)+1), so every product pairs equal k.
#include "fp8_device.h"
#include "launch.h"

namespace fp8lin {

namespace {

constexpr int kThreads = 256;
constexpr int BM = 128, BN = 128, BK = 128;

__device__ __forceinline__ float scale_at(int scaling, const float* __restrict__ s, int64_t rows,
                                          int64_t row, int64_t kb) {
  if (scaling == 0) return s[0];
  if (scaling == 1) return s[kb * rows + row];
  return s[kb * ((rows + 127) / 128) + row / 128];
}

// BLOCK: block-mode promotion per 128-wide K block.
// SB_COL: the B scale varies along N inside a tile (1x128 B operand).
template <int AF, int BF, bool BLOCK, bool SB_COL>
__global__ void __launch_bounds__(kThreads) k_gemm(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][2][BM * BK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t nk = (K + BK - 1) / BK;

  // ---- global -> register staging: 4 chunks of A and 4 of B per thread
  uint4 ra[4], rb[4];
  auto gload = [&](int64_t kt) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int row = it * 32 + (tid >> 3), ch = tid & 7;
      const int64_t k = kt * BK + ch * 16;
      const int64_t gm = m0 + row, gn = n0 + row;
      ra[it] = make_uint4(0, 0, 0, 0);
      rb[it] = make_uint4(0, 0, 0, 0);
      if (gm < M && k < K) ra[it] = *reinterpret_cast<const uint4*>(p.A + gm * p.lda + k);
      if (gn < N && k < K) rb[it] = *reinterpret_cast<const uint4*>(p.B + gn * p.ldb + k);
    }
  };
  auto lstore = [&](int stage) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int row = it * 32 + (tid >> 3), ch = tid & 7;
      const int off = row * BK + ((ch ^ (row & 7)) << 4);
      *reinterpret_cast<uint4*>(&smem[stage][0][off]) = ra[it];
      *reinterpret_cast<uint4*>(&smem[stage][1][off]) = rb[it];
    }
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int g = lane >> 4, l16 = lane & 15;
  // rows of this lane's outputs: tile i, entry r -> 16*i + 4*g + r (+ wave offset)
  const int64_t mrow0 = m0 + wm * 64 + 4 * g;
  const int64_t ncol0 = n0 + wn * 64 + l16;

  gload(0);
  lstore(0);
  __syncthreads();

  for (int64_t kt = 0; kt < nk; ++kt) {
    const int stage = (int)(kt & 1);
    if (kt + 1 < nk) gload(kt + 1);

    // per-block scales for this K block
    float srow[4][4], scol[4];
    if constexpr (BLOCK) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t m = mrow0 + 16 * i + r;
          srow[i][r] = scale_at(p.a_scaling, p.a_sinv, M, m < M ? m : M - 1, kt);
        }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = ncol0 + 16 * j;
        scol[j] = scale_at(p.b_scaling, p.b_sinv, N, n < N ? n : N - 1, kt);
      }
      if constexpr (!SB_COL) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) srow[i][r] *= scol[0];
      }
    }

    const uint8_t* As = smem[stage][0];
    const uint8_t* Bs = smem[stage][1];
    v8i af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 64 + 16 * i + l16;
      const uint4 lo = *reinterpret_cast<const uint4*>(As + row * BK + (((2 * g) ^ (row & 7)) << 4));
      const uint4 hi =
          *reinterpret_cast<const uint4*>(As + row * BK + (((2 * g + 1) ^ (row & 7)) << 4));
      af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                  (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wn * 64 + 16 * j + l16;
      const uint4 lo = *reinterpret_cast<const uint4*>(Bs + row * BK + (((2 * g) ^ (row & 7)) << 4));
      const uint4 hi =
          *reinterpret_cast<const uint4*>(Bs + row * BK + (((2 * g + 1) ^ (row & 7)) << 4));
      bf[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                  (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (BLOCK) {
          const v4f part = mfma<AF, BF>(af[i], bf[j], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if constexpr (SB_COL)
              acc[i][j][r] = __builtin_fmaf(part[r] * srow[i][r], scol[j], acc[i][j][r]);
            else
              acc[i][j][r] = __builtin_fmaf(part[r], srow[i][r], acc[i][j][r]);
          }
        } else {
          acc[i][j] = mfma<AF, BF>(af[i], bf[j], acc[i][j]);
        }
      }

    if (kt + 1 < nk) lstore(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: dequantise (per-tensor or per-row scales), round, store,
  // output amax
  const int64_t astr = p.a_scaling == 5 ? 1 : 0, bstr = p.b_scaling == 5 ? 1 : 0;
  uint32_t amax_bits = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = mrow0 + 16 * i + r, n = ncol0 + 16 * j;
        if (m >= M || n >= N) continue;
        float v = acc[i][j][r];
        if constexpr (!BLOCK) v = (v * p.a_sinv[m * astr]) * p.b_sinv[n * bstr];
        if (p.d_f32) {
          float* d = reinterpret_cast<float*>(p.D) + m * p.ldd + n;
          if (p.accumulate) v = *d + v;
          *d = v;
          const uint32_t b = __float_as_uint(v) & 0x7FFFFFFFu;
          amax_bits = b > amax_bits ? b : amax_bits;
        } else {
          const uint16_t h = f32_to_bf16_rne(v);
          reinterpret_cast<uint16_t*>(p.D)[m * p.ldd + n] = h;
          const uint32_t b = (uint32_t)(h & 0x7FFFu) << 16;
          amax_bits = b > amax_bits ? b : amax_bits;
        }
      }
  if (p.d_amax) {
    amax_bits = wave_max_u32(amax_bits);
    if (lane == 0 && amax_bits != 0u) atomic_max_bits(p.d_amax, amax_bits);
  }
}

// Zero output for K == 0 (or leave it when accumulating).
__global__ void k_zero_out(GemmParams p) {
  const int64_t total = p.M * p.N;
  uint32_t amax_bits = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / p.N, n = i - m * p.N;
    if (p.d_f32) {
      if (!p.accumulate) reinterpret_cast<float*>(p.D)[m * p.ldd + n] = 0.0f;
      if (p.d_amax) {
        const uint32_t b =
            __float_as_uint(reinterpret_cast<float*>(p.D)[m * p.ldd + n]) & 0x7FFFFFFFu;
        amax_bits = b > amax_bits ? b : amax_bits;
      }
    } else if (p.d_fp8) {
      reinterpret_cast<uint8_t*>(p.D)[m * p.ldd + n] = 0;
      if (p.D_t) p.D_t[n * p.ldt + m] = 0;
    } else {
      reinterpret_cast<uint16_t*>(p.D)[m * p.ldd + n] = 0;
    }
  }
  if (p.d_amax) {
    amax_bits = wave_max_u32(amax_bits);
    if ((threadIdx.x & 63) == 0 && amax_bits != 0u) atomic_max_bits(p.d_amax, amax_bits);
  }
}

template <int AF, int BF>
hipError_t launch_fmt(const GemmParams& p, hipStream_t s) {
  dim3 grid((unsigned)((p.N + BN - 1) / BN), (unsigned)((p.M + BM - 1) / BM));
  const bool block = !((p.a_scaling == 0 || p.a_scaling == 5) &&
                       (p.b_scaling == 0 || p.b_scaling == 5));
  const bool sb_col = p.b_scaling == 1;
  if (!block)
    hipLaunchKernelGGL((k_gemm<AF, BF, false, false>), grid, dim3(kThreads), 0, s, p);
  else if (sb_col)
    hipLaunchKernelGGL((k_gemm<AF, BF, true, true>), grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((k_gemm<AF, BF, true, false>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  if (p.d_amax && !p.amax_acc) {
    hipError_t e = launch_fill_u32(reinterpret_cast<uint32_t*>(p.d_amax), 1, 0u, s);
    if (e != hipSuccess) return e;
  }
  if (p.M == 0 || p.N == 0) return hipSuccess;
  if (p.K == 0) {
    int64_t blocks = (p.M * p.N + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_zero_out, dim3((unsigned)blocks), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  if (gemm_big_supported(p)) return launch_gemm_big(p, s);
  // this kernel promotes every block scale in FP32: power-of-two block
  // scales (codes 3, 4) are binary32 scales of the same layouts (1, 2)
  GemmParams q = p;
  if (q.a_scaling == 3 || q.a_scaling == 4) q.a_scaling -= 2;
  if (q.b_scaling == 3 || q.b_scaling == 4) q.b_scaling -= 2;
  if (q.a_fmt == 0 && q.b_fmt == 0) return launch_fmt<0, 0>(q, s);
  if (q.a_fmt == 1 && q.b_fmt == 0) return launch_fmt<1, 0>(q, s);
  if (q.a_fmt == 0 && q.b_fmt == 1) return launch_fmt<0, 1>(q, s);
  return launch_fmt<1, 1>(q, s);
}

}  // namespace fp8lin
