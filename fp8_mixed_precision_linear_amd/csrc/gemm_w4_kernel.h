// gemm_w4_kernel.h -- the FP8 GEMM on four wavefronts of 128 x 128
// (accumulators in the matrix unit's AGPRs) for per-tensor, per-row and
// power-of-two block scales; instantiated by gemm_w4.hip / gemm_w4_fp8out.hip
// (per-tensor and per-row; BF16 / FP32 and FP8 output) and gemm_w4_mx.hip /
// gemm_w4_mx_fp8out.hip (power-of-two block scales).
//
// Same contract as k_gemm_big (gemm_big_kernel.h, whose helpers and
// epilogue it shares): D = A . B^T, K-contiguous FP8 operands, FP32
// accumulation, per-tensor and per-row scales applied once in the epilogue
// ([MPG] "Mixed Precision LLM Training: The Complete Guide", "Transformer
// Engine internals > Delayed scaling"), power-of-two block scales inside
// the matrix instruction; the same 256 x 256 output tile, the same two LDS
// stages filled by buffer_load ... lds, the same swizzle and workgroup
// order.
//
// What differs is the wavefront layout and the step's schedule.  One
// wavefront per SIMD with a 128 x 128 tile reads every fragment once per
// step: 32 ds_read_b128 per 64 MFMAs, against 1.5 times those bytes for
// eight wavefronts of 128 x 64.  The step is split around its barrier:
//   row-tiles 0..3 go row by row, each reading the next row-tile's A
//   fragment after its first MFMA and one of row-tiles 4..7's after its
//   fifth;
//   then every read of the stage has been issued: wait for them and for this
//   wavefront's DMA of the other stage, barrier;
//   row-tiles 4..7 go column by column, so B column-tile j is free after its
//   fourth MFMA and is refilled from the next stage right then; two DMA
//   instructions of the step after next go between its MFMAs, one after
//   the first and one after the third.
// The next stage's 18 fragment reads and 16 DMA instructions thus spread
// over 32 MFMAs instead of following the barrier in a burst, which with the
// barrier's wait for the slowest wavefront cost 10-18% on the
// transformer-block shapes; every read or DMA instruction sits between two
// MFMAs (2-3% faster than issuing each group's reads and DMA together).
#pragma once

#include "gemm_big_kernel.h"

namespace fp8lin {

namespace {

constexpr int W4_THREADS = 256;
constexpr int W4_STAGE = A_BYTES + B_BYTES;   // 64 KB: A then B (block modes: + scale rows)
enum : int { W4_TENSOR = 0, W4_ROWS = 1, W4_MX = 2 };
// FP8 output: the epilogue in two passes of 64 rows (fewer codes live at a
// time; the column-major copy, 18 KB, and a 64-row row-major area, 8 KB,
// fit in the wavefront's 32 KB)
constexpr int W4_OUT8_PASSES = 2;

// KT: K is not a multiple of the step (chunks past K map to the
// out-of-range marker, step by step); OUT8: FP8 output quantised in the
// epilogue (codes, optional transposed copy, amax of the unquantised
// values).  MODE: W4_TENSOR, per-tensor scales; W4_ROWS, one scale per row
// of A (a_scaling 5) and / or of B (b_scaling 5), the other operand
// possibly per tensor, applied after the K sum ([MPG] "Per-row vs
// per-tensor scaling"); W4_MX + (A 1x128 ? 1 : 0) + (B 1x128 ? 2 : 0),
// power-of-two block scales (E8M0 codes) applied inside the matrix
// instruction, the accumulator staying in its C operand ([MPG] "DeepSeek
// FP8 training recipe in detail > Block-wise scaling at 128 granularity";
// a per-tensor operand's scale goes to the epilogue).
template <int AF, int BF, bool KT, bool OUT8, int MODE>
__global__ void __launch_bounds__(W4_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_gemm_w4(GemmParams p, int tiles_m, int tiles_n) {
  constexpr bool ROWS = MODE == W4_ROWS, MX = MODE >= W4_MX;
  constexpr bool SA_ROWS = MX && ((MODE - W4_MX) & 1), SB_COL = MX && ((MODE - W4_MX) & 2);
  static_assert(!(MX && KT), "block scales make K a multiple of the step");
  // a stage: A, B, then (block modes) 256 row scales of A and of B
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][MX ? STAGE : W4_STAGE];
  // per-row scales of the tile's 256 D rows and 256 D columns (rows clamped
  // into D for edge tiles), read in the epilogue
  __shared__ float rs_tab[ROWS ? BM + BN : 1];
  // block modes: per wavefront and K block, the E8M0 codes of the uniform
  // (128 x 128 or per-tensor) scales, A in bits 0-7, B in bits 8-15
  __shared__ float su_tab[MX ? 4 : 1][MX ? MAX_KB : 1];
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
  if constexpr (MODE == W4_TENSOR) {
    sa = p.a_sinv[0];
    sb = p.b_sinv[0];
  }
  if constexpr (MX) {   // a per-tensor operand's scale
    if (p.a_scaling == 0) sa = p.a_sinv[0];
    if (p.b_scaling == 0) sb = p.b_sinv[0];
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
  // block modes: the K block's 256 A row scales and 256 B column scales,
  // wavefront w fetching rows (columns) 64w .. 64w + 63 of each (rows past
  // the end read zeros); two instructions per wavefront and stage
  auto load_scales = [&](int kb, const uint8_t* base) {
    const uint32_t lb = lds_addr(base);
    if constexpr (SA_ROWS) {
      const i32x4 rs = make_rsrc(p.a_sinv + (int64_t)kb * M + m0, (uint32_t)(rows_a * 4));
      dma4(lb + SA_OFF + wave * 256, (uint32_t)(wave * 256 + lane * 4), rs);
    }
    if constexpr (SB_COL) {
      const i32x4 rs = make_rsrc(p.b_sinv + (int64_t)kb * N + n0, (uint32_t)(rows_b * 4));
      dma4(lb + SB_OFF + wave * 256, (uint32_t)(wave * 256 + lane * 4), rs);
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
  load_scales(0, lds[0]);
  if (nk > 1) {
#pragma unroll
    for (int q = 0; q < 16; ++q) load(1, lds[1], q);
    load_scales(1, lds[1]);
  }
  if constexpr (ROWS) {   // thread t: A's scale of D row m0 + t, then B's of column n0 + t
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t r = (h == 0 ? m0 : n0) + tid, lim = h == 0 ? M : N;
      const bool row_mode = (h == 0 ? p.a_scaling : p.b_scaling) == 5;
      rs_tab[h * BM + tid] = (h == 0 ? p.a_sinv : p.b_sinv)[row_mode ? (r < lim ? r : lim - 1) : 0];
    }
  }
  if constexpr (MX && !(SA_ROWS && SB_COL)) {
    // the uniform parts: the wavefront's 128 rows and 128 columns each sit
    // in one 128 x 128 block (1.0, code 127, for a per-tensor operand)
    const int64_t mb = min((m0 + wm * 128) / 128, (M + 127) / 128 - 1);
    const int64_t nb = min((n0 + wn * 128) / 128, (N + 127) / 128 - 1);
    for (int k = lane; k < nk; k += 64) {
      int ea = 127, eb = 127;
      if constexpr (!SA_ROWS)
        if (p.a_scaling != 0) ea = e8m0_of(p.a_sinv[k * ((M + 127) / 128) + mb]);
      if constexpr (!SB_COL)
        if (p.b_scaling != 0) eb = e8m0_of(p.b_sinv[k * ((N + 127) / 128) + nb]);
      su_tab[wave][k] = __uint_as_float((uint32_t)ea | ((uint32_t)eb << 8));
    }
  }
  // stage 0 done (in the block modes up to 2 more DMA instructions per
  // stage: the wait then covers part of stage 1 as well)
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
  // block modes: the step's scales of A's row-tiles (lane l16: row
  // 16 i + l16) and of B's column-tiles (column 16 j + l16), kept as read;
  // their E8M0 codes are taken at the MFMA, long after the read returned
  float ea[8], eb[8];
  auto ea_of = [&](const uint8_t* S, int i) {
    return reinterpret_cast<const float*>(S + SA_OFF)[wm * 128 + 16 * i + l16];
  };
  auto eb_of = [&](const uint8_t* S, int j) {
    return reinterpret_cast<const float*>(S + SB_OFF)[wn * 128 + 16 * j + l16];
  };
  if constexpr (SA_ROWS) {
#pragma unroll
    for (int i = 0; i < 8; ++i) ea[i] = ea_of(lds[0], i);
  }
  if constexpr (SB_COL) {
#pragma unroll
    for (int j = 0; j < 8; ++j) eb[j] = eb_of(lds[0], j);
  }
  // one MFMA: plain, or with the block codes of row-tile i and column-tile j
  auto mm = [&](const v8i& bj, const v8i& ai, const v4f& c, int i, int j, uint32_t eu) -> v4f {
    if constexpr (MX)
      return mfma_mx<BF, AF>(bj, ai, c, SB_COL ? e8m0_of(eb[j]) : (int)((eu >> 8) & 0xFFu),
                             SA_ROWS ? e8m0_of(ea[i]) : (int)(eu & 0xFFu));
    else
      return mfma<BF, AF>(bj, ai, c);
  };

  // One K step on stage X, with B's fragments and row-tile 0's A fragment
  // in registers; Y is the next step's stage.  The scheduling barriers keep
  // the compiler to this order.
  auto step = [&](auto dmatag, auto nexttag, const uint8_t* X, const uint8_t* Y, int kb) {
    constexpr bool DMA = decltype(dmatag)::value;    // issue the DMA of step kb + 2
    constexpr bool NEXT = decltype(nexttag)::value;  // read step kb + 1's fragments
    uint32_t eu = 0;
    if constexpr (MX && !(SA_ROWS && SB_COL)) eu = __float_as_uint(su_tab[wave][kb]);
    __builtin_amdgcn_sched_barrier(0);
    // row-tiles 0..3, row by row: the next row-tile's A fragment is read
    // after this row's first MFMA, row-tile i + 4's after its fifth
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j == 1 && i < 3) a[(i + 1) & 1] = frag(X, ar + 16 * (i + 1), g);
        if (j == 5) h[i] = frag(X, ar + 16 * (i + 4), g);
        if (j == 1 || j == 5) __builtin_amdgcn_sched_barrier(0);
        acc[i][j] = mm(b[j], a[i & 1], acc[i][j], i, j, eu);
        if (j == 0 || j == 4) __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NEXT) {
      // every read of X is issued: once they and this wavefront's DMA of Y
      // are done everywhere, Y may be read and X refilled
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      a[0] = frag(Y, ar, g);
      if constexpr (SA_ROWS) {   // row-tiles 0..3 are done with theirs
#pragma unroll
        for (int i = 0; i < 4; ++i) ea[i] = ea_of(Y, i);
      }
    }
    // row-tiles 4..7, column by column: two DMA instructions of step kb + 2
    // after the column's first and third MFMA, then B column-tile j, free
    // after its fourth, refilled from the next stage
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int i = 4; i < 8; ++i) {
        acc[i][j] = mm(b[j], h[i - 4], acc[i][j], i, j, eu);
        if constexpr (DMA) {
          if (i == 4 || i == 6) {
            __builtin_amdgcn_sched_barrier(0);
            load(kb + 2, X, 2 * j + (i - 4) / 2);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      if constexpr (NEXT) b[j] = frag(Y + A_BYTES, br + 16 * j, g);
      if constexpr (SB_COL && NEXT) eb[j] = eb_of(Y, j);
      if constexpr (DMA) {
        if (j == 7) load_scales(kb + 2, X);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (SA_ROWS && NEXT) {
#pragma unroll
      for (int i = 4; i < 8; ++i) ea[i] = ea_of(Y, i);
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
  // With per-row or block scales every output is checked.
  constexpr int QAB = (AF == 0 ? 9 : 16) + (BF == 0 ? 9 : 16);
  const float lo = (__builtin_ldexpf(1.0f, -QAB) * __builtin_fabsf(sa)) * __builtin_fabsf(sb);
  const bool may_sub = MODE != W4_TENSOR || !(lo >= 1.17549435e-38f);   // NaN scales: check
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

template <int AF, int BF, bool OUT8, int MODE>
hipError_t launch_w4_k(const GemmParams& p, hipStream_t s) {
  const int tiles_m = (int)((p.M + BM - 1) / BM), tiles_n = (int)((p.N + BN - 1) / BN);
  const dim3 grid((unsigned)(tiles_m * tiles_n)), block(W4_THREADS);
  if constexpr (MODE >= W4_MX)   // block scales: K is a multiple of the step
    hipLaunchKernelGGL((k_gemm_w4<AF, BF, false, OUT8, MODE>), grid, block, 0, s, p, tiles_m, tiles_n);
  else if (p.K % BK == 0)
    hipLaunchKernelGGL((k_gemm_w4<AF, BF, false, OUT8, MODE>), grid, block, 0, s, p, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL((k_gemm_w4<AF, BF, true, OUT8, MODE>), grid, block, 0, s, p, tiles_m, tiles_n);
  return hipGetLastError();
}

// MX = false: per-tensor or per-row scales; MX = true: power-of-two block
// scales (codes 3 / 4) or per-tensor on each operand, at least one blocked.
template <int AF, int BF, bool OUT8, bool MX>
hipError_t launch_w4(const GemmParams& p, hipStream_t s) {
  if constexpr (MX) {
    const bool ra = p.a_scaling == 3, cb = p.b_scaling == 3;   // 1x128 tiles
    if (ra && cb) return launch_w4_k<AF, BF, OUT8, W4_MX + 3>(p, s);
    if (ra) return launch_w4_k<AF, BF, OUT8, W4_MX + 1>(p, s);
    if (cb) return launch_w4_k<AF, BF, OUT8, W4_MX + 2>(p, s);
    return launch_w4_k<AF, BF, OUT8, W4_MX>(p, s);
  } else {
    return p.a_scaling == 5 || p.b_scaling == 5 ? launch_w4_k<AF, BF, OUT8, W4_ROWS>(p, s)
                                                : launch_w4_k<AF, BF, OUT8, W4_TENSOR>(p, s);
  }
}

template <bool OUT8, bool MX>
hipError_t launch_w4_out(const GemmParams& p, hipStream_t s) {
  if (p.a_fmt == 0 && p.b_fmt == 0) return launch_w4<0, 0, OUT8, MX>(p, s);
  if (p.a_fmt == 1 && p.b_fmt == 0) return launch_w4<1, 0, OUT8, MX>(p, s);
  if (p.a_fmt == 0 && p.b_fmt == 1) return launch_w4<0, 1, OUT8, MX>(p, s);
  return launch_w4<1, 1, OUT8, MX>(p, s);
}

}  // namespace

}  // namespace fp8lin
