// gemm_w4_kernel.h -- the per-tensor-scaled FP8 GEMM on four wavefronts of
// 128 x 128 (accumulators in the matrix unit's AGPRs); instantiated by
// gemm_w4.hip (BF16 / FP32 output) and gemm_w4_fp8out.hip (FP8 output).
//
// Same contract as k_gemm_big (gemm_big_kernel.h, whose helpers and
// epilogue it shares): D = A . B^T, K-contiguous FP8 operands, FP32
// accumulation, the two per-tensor scales applied once in the epilogue
// ([MPG] "Mixed Precision LLM Training: The Complete Guide", "Transformer
// Engine internals > Delayed scaling"), the same 256 x 256 output tile, the
// same two 64 KB LDS stages filled by buffer_load ... lds, the same swizzle
// and workgroup order.
//
// What differs is the wavefront layout and the step's schedule.  One
// wavefront per SIMD with a 128 x 128 tile reads every fragment once per
// step: 32 ds_read_b128 per 64 MFMAs, against 1.5 times those bytes for
// eight wavefronts of 128 x 64.  The step is split around its barrier:
//   row-tiles 0..3 go row by row, each reading the next row-tile's A
//   fragment, and one of row-tiles 4..7's, ahead of its MFMAs;
//   then every read of the stage has been issued: wait for them and for this
//   wavefront's DMA of the other stage, barrier;
//   row-tiles 4..7 go column by column, so B column-tile j is free after its
//   fourth MFMA and is refilled from the next stage right then, with two
//   DMA instructions of the step after next beside it.
// The next stage's 18 fragment reads and 16 DMA instructions thus spread
// over 32 MFMAs instead of following the barrier in a burst, which with the
// barrier's wait for the slowest wavefront cost 10-18% on the
// transformer-block shapes.
#pragma once

#include "gemm_big_kernel.h"

namespace fp8lin {

namespace {

constexpr int W4_THREADS = 256;
constexpr int W4_STAGE = A_BYTES + B_BYTES;   // 64 KB: A then B, no scale rows
// FP8 output: the epilogue in two passes of 64 rows (fewer codes live at a
// time; the column-major copy, 18 KB, and a 64-row row-major area, 8 KB,
// fit in the wavefront's 32 KB)
constexpr int W4_OUT8_PASSES = 2;

// KT: K is not a multiple of the step (chunks past K map to the
// out-of-range marker, step by step); OUT8: FP8 output quantised in the
// epilogue (codes, optional transposed copy, amax of the unquantised
// values); ROWS: one scale per row of A (a_scaling 5) and / or of B
// (b_scaling 5), the other operand possibly per tensor, applied after the
// K sum ([MPG] "Per-row vs per-tensor scaling").
template <int AF, int BF, bool KT, bool OUT8, bool ROWS>
__global__ void __launch_bounds__(W4_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_gemm_w4(GemmParams p, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][W4_STAGE];
  // per-row scales of the tile's 256 D rows and 256 D columns (rows clamped
  // into D for edge tiles), read in the epilogue
  __shared__ float rs_tab[ROWS ? BM + BN : 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int nk = (int)((K + BK - 1) / BK);

  // ---- tile id: contiguous runs per XCD, grouped by 8 tile-rows
  const int nblk = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int group = bid / (GROUP_M * tiles_n);
  const int first_m = group * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int in_group = bid - group * GROUP_M * tiles_n;
  const int tm = first_m + in_group % gm, tn = in_group / gm;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int64_t rows_a = min((int64_t)BM, M - m0), rows_b = min((int64_t)BN, N - n0);
  const i32x4 ra = make_rsrc(p.A + m0 * p.lda, (uint32_t)(rows_a * p.lda));
  const i32x4 rb = make_rsrc(p.B + n0 * p.ldb, (uint32_t)(rows_b * p.ldb));
  const int lda = (int)p.lda, ldb = (int)p.ldb;

  // the epilogue's scales, read ahead of the first DMA (its wait covers them)
  float sa = 1.0f, sb = 1.0f;
  if constexpr (!ROWS) {
    sa = p.a_sinv[0];
    sb = p.b_sinv[0];
  }
  float so = 1.0f;
  if constexpr (OUT8) so = p.d_scale[0];

  // ---- DMA: wavefront w fills rows 64w .. 64w + 63 of A and of B, 8 rows
  // per instruction; lane l lands in row 8 it + l / 8 of the group, stored
  // chunk l % 8, and fetches the K chunk the swizzle puts there, which
  // depends only on the parity of it.  The row offset stays in the lane
  // offset, so rows past the operand's end fail the buffer's range check
  // and read zeros; with K a multiple of the step the step's K offset rides
  // in the scalar offset, otherwise chunks past K get the out-of-range
  // marker.
  uint32_t ro[2][8], kcl[2];
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int row = 64 * wave + 8 * it + (lane >> 3);
    ro[0][it] = (uint32_t)(row * lda);
    ro[1][it] = (uint32_t)(row * ldb);
  }
#pragma unroll
  for (int par = 0; par < 2; ++par)
    kcl[par] = (uint32_t)(16 * ((lane & 7) ^ swz(64 * wave + 8 * par + (lane >> 3))));
  auto load = [&](int kb, const uint8_t* base, int q) {   // q: 0..7 A, 8..15 B
    const int o = q >> 3, it = q & 7;
    const uint32_t dst = lds_addr(base) + (o ? A_BYTES : 0) + (64 * wave + 8 * it) * BK;
    if constexpr (!KT) {
      dma16s(dst, ro[o][it] + kcl[it & 1], o ? rb : ra, (uint32_t)(kb * BK));
    } else {
      const int kc = kb * BK + (int)kcl[it & 1];
      dma16(dst, kc < (int)K ? ro[o][it] + (uint32_t)kc : kOOB, o ? rb : ra);
    }
  };

  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // the first two stages go out together; wait for the first (16 DMA
  // instructions per stage and wavefront, counted down in issue order)
#pragma unroll
  for (int q = 0; q < 16; ++q) load(0, lds[0], q);
  if (nk > 1) {
#pragma unroll
    for (int q = 0; q < 16; ++q) load(1, lds[1], q);
  }
  if constexpr (ROWS) {   // thread t: A's scale of D row m0 + t, then B's of column n0 + t
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t r = (h == 0 ? m0 : n0) + tid, lim = h == 0 ? M : N;
      const bool row_mode = (h == 0 ? p.a_scaling : p.b_scaling) == 5;
      rs_tab[h * BM + tid] = (h == 0 ? p.a_sinv : p.b_sinv)[row_mode ? (r < lim ? r : lim - 1) : 0];
    }
  }
  if (nk > 1) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // Lane (g, l16) of the transposed MFMA (B is its first operand) holds D
  // row 16 i + l16, columns 16 j + 4 g .. +3 of the wavefront's tile.
  const int ar = wm * 128 + l16, br = wn * 128 + l16;
  v8i b[8], a[2], h[4];
#pragma unroll
  for (int j = 0; j < 8; ++j) b[j] = frag(lds[0] + A_BYTES, br + 16 * j, g);
  a[0] = frag(lds[0], ar, g);

  // One K step on stage X, with B's fragments and row-tile 0's A fragment
  // in registers; Y is the next step's stage.  The scheduling barriers keep
  // the compiler to this order.
  auto step = [&](auto dmatag, auto nexttag, const uint8_t* X, const uint8_t* Y, int kb) {
    constexpr bool DMA = decltype(dmatag)::value;    // issue the DMA of step kb + 2
    constexpr bool NEXT = decltype(nexttag)::value;  // read step kb + 1's fragments
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < 3) a[(i + 1) & 1] = frag(X, ar + 16 * (i + 1), g);
      h[i] = frag(X, ar + 16 * (i + 4), g);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = mfma<BF, AF>(b[j], a[i & 1], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NEXT) {
      // every read of X is issued: once they and this wavefront's DMA of Y
      // are done everywhere, Y may be read and X refilled
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      a[0] = frag(Y, ar, g);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int i = 4; i < 8; ++i) acc[i][j] = mfma<BF, AF>(b[j], h[i - 4], acc[i][j]);
      if constexpr (NEXT) b[j] = frag(Y + A_BYTES, br + 16 * j, g);
      if constexpr (DMA) {
        load(kb + 2, X, 2 * j);
        load(kb + 2, X, 2 * j + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const std::true_type T{};
  const std::false_type F{};
  int kb = 0;
  for (; kb + 2 < nk; ++kb) step(T, T, lds[kb & 1], lds[(kb + 1) & 1], kb);
  if (kb + 1 < nk) {
    step(F, T, lds[kb & 1], lds[(kb + 1) & 1], kb);
    ++kb;
  }
  step(F, F, lds[kb & 1], lds[kb & 1], kb);

  // ---- epilogue (k_gemm_big's, for 128 x 128 wavefront tiles and 32 KB of
  // staging per wavefront).  With per-tensor scales every nonzero
  // accumulator is a multiple of 2^-(qa + qb) (the two formats' smallest
  // subnormal steps), so if that minimum dequantises to a normal binary32,
  // no output can be subnormal.
  // With per-row scales every output is checked.
  constexpr int QAB = (AF == 0 ? 9 : 16) + (BF == 0 ? 9 : 16);
  const float lo = (__builtin_ldexpf(1.0f, -QAB) * __builtin_fabsf(sa)) * __builtin_fabsf(sb);
  const bool may_sub = ROWS || !(lo >= 1.17549435e-38f);   // NaN scales: check
  auto deq = [&](int i, int j, int q, float x) -> float {
    if constexpr (ROWS)
      return (x * rs_tab[wm * 128 + 16 * i + l16]) * rs_tab[BM + wn * 128 + 16 * j + 4 * g + q];
    else
      return (x * sa) * sb;
  };
  const int esz = OUT8 ? 1 : (p.d_f32 ? 4 : 2);
  const bool staged = (m0 + BM <= M) && (n0 + BN <= N) && ((p.ldd * esz) % 16 == 0) &&
                      ((reinterpret_cast<uintptr_t>(p.D) & 15u) == 0) &&
                      (!OUT8 || p.D_t == nullptr ||
                       ((p.ldt % 16 == 0) && ((reinterpret_cast<uintptr_t>(p.D_t) & 15u) == 0)));
  uint32_t amax_bits;
  if (staged) {
    __syncthreads();   // every wavefront is done reading both stages
    uint8_t* wl = &lds[0][0] + wave * 32768;
    if constexpr (OUT8)
      amax_bits = store_staged8<8, 8, W4_OUT8_PASSES>(p, acc, deq, so, m0 + wm * 128, n0 + wn * 128, lane, wl);
    else
      amax_bits = store_staged<8, 8, 32768>(p, acc, deq, may_sub, m0 + wm * 128, n0 + wn * 128,
                                            lane, wl);
  } else {
    amax_bits = store_edge<8, 8, OUT8>(p, acc, deq, so, m0 + wm * 128, n0 + wn * 128, lane);
  }
  if (p.d_amax) workgroup_amax<4>(p.d_amax, amax_bits, lane, wave);
}

template <int AF, int BF, bool OUT8, bool ROWS>
hipError_t launch_w4_k(const GemmParams& p, hipStream_t s) {
  const int tiles_m = (int)((p.M + BM - 1) / BM), tiles_n = (int)((p.N + BN - 1) / BN);
  const dim3 grid((unsigned)(tiles_m * tiles_n)), block(W4_THREADS);
  if (p.K % BK == 0)
    hipLaunchKernelGGL((k_gemm_w4<AF, BF, false, OUT8, ROWS>), grid, block, 0, s, p, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL((k_gemm_w4<AF, BF, true, OUT8, ROWS>), grid, block, 0, s, p, tiles_m, tiles_n);
  return hipGetLastError();
}

template <int AF, int BF, bool OUT8>
hipError_t launch_w4(const GemmParams& p, hipStream_t s) {
  return p.a_scaling == 5 || p.b_scaling == 5 ? launch_w4_k<AF, BF, OUT8, true>(p, s)
                                              : launch_w4_k<AF, BF, OUT8, false>(p, s);
}

template <bool OUT8>
hipError_t launch_w4_out(const GemmParams& p, hipStream_t s) {
  if (p.a_fmt == 0 && p.b_fmt == 0) return launch_w4<0, 0, OUT8>(p, s);
  if (p.a_fmt == 1 && p.b_fmt == 0) return launch_w4<1, 0, OUT8>(p, s);
  if (p.a_fmt == 0 && p.b_fmt == 1) return launch_w4<0, 1, OUT8>(p, s);
  return launch_w4<1, 1, OUT8>(p, s);
}

}  // namespace

}  // namespace fp8lin
