// cast_block_kernels.hip -- block-wise FP8 quantisation on gfx950.
//
// [MPG] = "Mixed Precision LLM Training: The Complete Guide",
//   "DeepSeek FP8 training recipe in detail > Block-wise scaling at 128
//   granularity": one scale per 128x128 weight block and per 128-element
//   activation segment, computed on the fly and stored next to the data.
//
// One workgroup quantises one 128x128 tile of x from a single bf16 read:
//   1x128   : y   gets one scale per (row, 128 columns)      -> sinv  [cb][r]
//             y_t gets one scale per (column, 128 rows) (the token-axis
//             tiles of the transposed operand)               -> sinv_t[rb][c]
//   128x128 : one scale per tile; y_t is the byte transpose of y.
// Per tile: amax (exact packed 16-bit max of |x|), scale = fl32(fmax/amax)
// (1 for an all-zero tile), scale_inv = fl32(1/scale), then the saturating
// RNE cast of the per-tensor kernels with that scale.
#include "fp8_device.h"
#include "launch.h"

namespace fp8lin {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Halfwise unsigned 16-bit maximum of two packed pairs.
__device__ __forceinline__ uint32_t pk_umax(uint32_t a, uint32_t b) {
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, a),
                                                                __builtin_bit_cast(us2, b)));
}

// Binary32 pattern of max |x| over the two bf16 halves of a dword.
__device__ __forceinline__ uint32_t absmax2(uint32_t w) {
  uint32_t lo = (w & 0x7FFFu) << 16, hi = (w & 0x7FFF0000u);
  return umax(lo, hi);
}

// Scale for one tile from its amax bits (1 for all-zero / non-finite);
// P2: the power-of-two (exponent-bias) rule.
template <int FMT, bool P2>
__device__ __forceinline__ void tile_scale(uint32_t amax_bits, float& s, float& si) {
  s = 1.0f;
  si = 1.0f;
  if constexpr (P2) pow2_scale_from_amax(__uint_as_float(amax_bits), Fmt<FMT>::max, 0, s, si);
  else scale_from_amax(__uint_as_float(amax_bits), Fmt<FMT>::max, 0, s, si);
}

// Store the transposed tile from registers: w[i][j] holds the codes of row
// 4*rg+i, columns 16*cg+4j..+3.  Same LDS layout and swizzle as the
// per-tensor cast-transpose.
__device__ __forceinline__ void store_transposed(uint8_t* lds, const uint32_t (&w)[4][4], int cg,
                                                 int rg, int t, int64_t r0, int64_t c0,
                                                 int64_t rows, int64_t cols,
                                                 uint8_t* __restrict__ yt) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t t0, t1, t2, t3;
    transpose4x4(w[0][j], w[1][j], w[2][j], w[3][j], t0, t1, t2, t3);
    const uint32_t tv[4] = {t0, t1, t2, t3};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = 16 * cg + 4 * j + k;
      const int phys = (rg >> 2) ^ ((c >> 4) & 7);
      *reinterpret_cast<uint32_t*>(lds + c * 128 + phys * 16 + (rg & 3) * 4) = tv[k];
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = it * kThreads + t;
    const int c = idx >> 3, ch = idx & 7;
    const int phys = ch ^ ((c >> 4) & 7);
    const int64_t gc = c0 + c, gr = r0 + 16 * ch;
    if (gc < cols && gr < rows) {
      uint4 v = *reinterpret_cast<const uint4*>(lds + c * 128 + phys * 16);
      st_out16(v, (yt + gc * rows + gr));
    }
  }
}

// ---------------------------------------------------------------------
// Tiled kernel: rows % 16 == 0 and cols % 16 == 0.  Thread t owns rows
// 4*(t/8)..+3 and columns 16*(t%8)..+15 of the tile, held as raw bf16.
// ---------------------------------------------------------------------
template <int FMT, int TILE, bool WANT_Y, bool WANT_T, bool P2>
__global__ void __launch_bounds__(kThreads)
    k_cast_block(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                 uint8_t* __restrict__ y, float* __restrict__ sinv, uint8_t* __restrict__ yt,
                 float* __restrict__ sinv_t) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[128 * 128];
  __shared__ uint32_t red[4][128];     // per-wave partial maxima
  __shared__ float col_s[128];         // per-column scales (1x128 transposed copy)
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int cg = t & 7, rg = t >> 3;
  const int64_t rb = blockIdx.y, cb = blockIdx.x;
  const int64_t r0 = rb * 128, c0 = cb * 128;
  const int64_t nrb = (rows + 127) / 128, ncb = (cols + 127) / 128;
  const int64_t cbase = c0 + 16 * cg;
  const bool col_ok = cbase < cols;

  uint4 v[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = r0 + 4 * rg + i;
    v[i][0] = make_uint4(0, 0, 0, 0);
    v[i][1] = make_uint4(0, 0, 0, 0);
    if (col_ok && r < rows) {
      const uint4* p = reinterpret_cast<const uint4*>(x + r * cols + cbase);
      v[i][0] = ld_nt16(p);
      v[i][1] = ld_nt16(p + 1);
    }
  }

  uint32_t w[4][4];
  if constexpr (TILE == 2) {
    // ---- one scale for the whole 128x128 tile
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m = absmax_pk(m, v[i][0].x); m = absmax_pk(m, v[i][0].y);
      m = absmax_pk(m, v[i][0].z); m = absmax_pk(m, v[i][0].w);
      m = absmax_pk(m, v[i][1].x); m = absmax_pk(m, v[i][1].y);
      m = absmax_pk(m, v[i][1].z); m = absmax_pk(m, v[i][1].w);
    }
    uint32_t mb = wave_max_u32(absmax_fold(m));
    if (lane == 0) red[wave][0] = mb;
    __syncthreads();
    mb = umax(umax(red[0][0], red[1][0]), umax(red[2][0], red[3][0]));
    float s, si;
    tile_scale<FMT, P2>(mb, s, si);
    if (t == 0) {
      if (sinv) sinv[cb * nrb + rb] = si;
      if (sinv_t) sinv_t[rb * ncb + cb] = si;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint2 qa = cvt8_bf16<FMT>(v[i][0], s);
      uint2 qb = cvt8_bf16<FMT>(v[i][1], s);
      w[i][0] = qa.x; w[i][1] = qa.y; w[i][2] = qb.x; w[i][3] = qb.y;
      const int64_t r = r0 + 4 * rg + i;
      if (WANT_Y && col_ok && r < rows)
        st_out16(make_uint4(qa.x, qa.y, qb.x, qb.y),
                                    reinterpret_cast<uint4*>(y + r * cols + cbase));
    }
    if (WANT_T) store_transposed(lds, w, cg, rg, t, r0, c0, rows, cols, yt);
  } else {
    // ---- 1x128 along rows: reduce across the 8 lanes that share a row
    if constexpr (WANT_Y) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t m = 0;
        m = absmax_pk(m, v[i][0].x); m = absmax_pk(m, v[i][0].y);
        m = absmax_pk(m, v[i][0].z); m = absmax_pk(m, v[i][0].w);
        m = absmax_pk(m, v[i][1].x); m = absmax_pk(m, v[i][1].y);
        m = absmax_pk(m, v[i][1].z); m = absmax_pk(m, v[i][1].w);
        uint32_t mb = absmax_fold(m);
        mb = umax(mb, __shfl_xor(mb, 1, 64));
        mb = umax(mb, __shfl_xor(mb, 2, 64));
        mb = umax(mb, __shfl_xor(mb, 4, 64));
        float s, si;
        tile_scale<FMT, P2>(mb, s, si);
        const int64_t r = r0 + 4 * rg + i;
        if (cg == 0 && r < rows) sinv[cb * rows + r] = si;
        if (col_ok && r < rows) {
          uint2 qa = cvt8_bf16<FMT>(v[i][0], s);
          uint2 qb = cvt8_bf16<FMT>(v[i][1], s);
          st_out16(make_uint4(qa.x, qa.y, qb.x, qb.y),
                                      reinterpret_cast<uint4*>(y + r * cols + cbase));
        }
      }
    }
    // ---- 1x128 along columns (token axis) for the transposed copy
    if constexpr (WANT_T) {
      // column maxima as packed 16-bit pairs: dword j holds |x| of columns
      // 2j (low half) and 2j+1 (high half); bf16 magnitudes order like
      // their bit patterns, so one packed max per row and dword
      uint32_t cp[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) m = absmax_pk(m, (&v[i][0].x)[j]);
        cp[j] = m;
      }
      // across the 8 row groups of this wavefront (lanes with equal cg)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t m = cp[j];
        m = pk_umax(m, __shfl_xor(m, 8, 64));
        m = pk_umax(m, __shfl_xor(m, 16, 64));
        m = pk_umax(m, __shfl_xor(m, 32, 64));
        cp[j] = m;
      }
      if (lane < 8) {   // unpacked: binary32 patterns of the bf16 maxima
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          red[wave][16 * cg + 2 * j] = (cp[j] & 0xFFFFu) << 16;
          red[wave][16 * cg + 2 * j + 1] = cp[j] & 0xFFFF0000u;
        }
      }
      __syncthreads();
      if (t < 128) {
        const uint32_t mb = umax(umax(red[0][t], red[1][t]), umax(red[2][t], red[3][t]));
        float s, si;
        tile_scale<FMT, P2>(mb, s, si);
        col_s[t] = s;
        if (c0 + t < cols) sinv_t[rb * cols + c0 + t] = si;
      }
      __syncthreads();
      float sc[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) sc[k] = col_s[16 * cg + k];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t d0 = (&v[i][0].x)[2 * j], d1 = (&v[i][0].x)[2 * j + 1];
          w[i][j] = cvt4<FMT>(bf16_lo(d0) * sc[4 * j], bf16_hi(d0) * sc[4 * j + 1],
                              bf16_lo(d1) * sc[4 * j + 2], bf16_hi(d1) * sc[4 * j + 3]);
        }
      }
      store_transposed(lds, w, cg, rg, t, r0, c0, rows, cols, yt);
    }
  }
}

// ---------------------------------------------------------------------
// Generic kernel (any rows, cols): one workgroup per 128x128 tile; thread
// t < 128 handles row t (1x128 rows) or column t (token-axis tiles) of the
// tile with scalar loops; 128x128 reduces over the whole tile.
// ---------------------------------------------------------------------
template <int FMT, int TILE, bool P2>
__global__ void __launch_bounds__(kThreads)
    k_cast_block_generic(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                         uint8_t* __restrict__ y, float* __restrict__ sinv,
                         uint8_t* __restrict__ yt, float* __restrict__ sinv_t) {
  __shared__ uint32_t red[kThreads / 64];
  const int t = threadIdx.x;
  const int64_t rb = blockIdx.y, cb = blockIdx.x;
  const int64_t r0 = rb * 128, c0 = cb * 128;
  const int64_t r1 = r0 + 128 < rows ? r0 + 128 : rows, c1 = c0 + 128 < cols ? c0 + 128 : cols;
  const int64_t nrb = (rows + 127) / 128, ncb = (cols + 127) / 128;
  if constexpr (TILE == 2) {
    uint32_t m = 0;
    for (int64_t idx = t; idx < (r1 - r0) * (c1 - c0); idx += kThreads) {
      const int64_t r = r0 + idx / (c1 - c0), c = c0 + idx % (c1 - c0);
      m = umax(m, (uint32_t)(x[r * cols + c] & 0x7FFFu) << 16);
    }
    m = wave_max_u32(m);
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    m = umax(umax(red[0], red[1]), umax(red[2], red[3]));
    float s, si;
    tile_scale<FMT, P2>(m, s, si);
    if (t == 0) {
      if (sinv) sinv[cb * nrb + rb] = si;
      if (sinv_t) sinv_t[rb * ncb + cb] = si;
    }
    for (int64_t idx = t; idx < (r1 - r0) * (c1 - c0); idx += kThreads) {
      const int64_t r = r0 + idx / (c1 - c0), c = c0 + idx % (c1 - c0);
      const uint8_t q = (uint8_t)(cvt4<FMT>(__uint_as_float((uint32_t)x[r * cols + c] << 16) * s,
                                            0.f, 0.f, 0.f) & 0xFFu);
      if (y) y[r * cols + c] = q;
      if (yt) yt[c * rows + r] = q;
    }
  } else {
    if (y && t < r1 - r0) {
      const int64_t r = r0 + t;
      uint32_t m = 0;
      for (int64_t c = c0; c < c1; ++c) m = umax(m, (uint32_t)(x[r * cols + c] & 0x7FFFu) << 16);
      float s, si;
      tile_scale<FMT, P2>(m, s, si);
      sinv[cb * rows + r] = si;
      for (int64_t c = c0; c < c1; ++c)
        y[r * cols + c] = (uint8_t)(cvt4<FMT>(__uint_as_float((uint32_t)x[r * cols + c] << 16) * s,
                                              0.f, 0.f, 0.f) & 0xFFu);
    }
    if (yt && t < c1 - c0) {
      const int64_t c = c0 + t;
      uint32_t m = 0;
      for (int64_t r = r0; r < r1; ++r) m = umax(m, (uint32_t)(x[r * cols + c] & 0x7FFFu) << 16);
      float s, si;
      tile_scale<FMT, P2>(m, s, si);
      sinv_t[rb * cols + c] = si;
      for (int64_t r = r0; r < r1; ++r)
        yt[c * rows + r] = (uint8_t)(cvt4<FMT>(__uint_as_float((uint32_t)x[r * cols + c] << 16) * s,
                                               0.f, 0.f, 0.f) & 0xFFu);
    }
  }
}

template <int FMT, int TILE, bool P2>
hipError_t launch_block_t(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* y, float* sinv,
                          uint8_t* yt, float* sinv_t, hipStream_t s) {
  dim3 grid((unsigned)((cols + 127) / 128), (unsigned)((rows + 127) / 128));
  if (rows % 16 == 0 && cols % 16 == 0) {
    if (y && yt)
      hipLaunchKernelGGL((k_cast_block<FMT, TILE, true, true, P2>), grid, dim3(kThreads), 0, s, x,
                         rows, cols, y, sinv, yt, sinv_t);
    else if (y)
      hipLaunchKernelGGL((k_cast_block<FMT, TILE, true, false, P2>), grid, dim3(kThreads), 0, s, x,
                         rows, cols, y, sinv, yt, sinv_t);
    else
      hipLaunchKernelGGL((k_cast_block<FMT, TILE, false, true, P2>), grid, dim3(kThreads), 0, s, x,
                         rows, cols, y, sinv, yt, sinv_t);
  } else {
    hipLaunchKernelGGL((k_cast_block_generic<FMT, TILE, P2>), grid, dim3(kThreads), 0, s, x, rows,
                       cols, y, sinv, yt, sinv_t);
  }
  return hipGetLastError();
}

}  // namespace

template <bool P2>
hipError_t launch_block_p(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int tile,
                          uint8_t* y, float* sinv, uint8_t* y_t, float* sinv_t, hipStream_t s) {
  if (fmt == 0)
    return tile == 2 ? launch_block_t<0, 2, P2>(x, rows, cols, y, sinv, y_t, sinv_t, s)
                     : launch_block_t<0, 1, P2>(x, rows, cols, y, sinv, y_t, sinv_t, s);
  return tile == 2 ? launch_block_t<1, 2, P2>(x, rows, cols, y, sinv, y_t, sinv_t, s)
                   : launch_block_t<1, 1, P2>(x, rows, cols, y, sinv, y_t, sinv_t, s);
}

hipError_t launch_cast_block(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int tile,
                             int pow2, uint8_t* y, float* sinv, uint8_t* y_t, float* sinv_t,
                             hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  return pow2 ? launch_block_p<true>(x, rows, cols, fmt, tile, y, sinv, y_t, sinv_t, s)
              : launch_block_p<false>(x, rows, cols, fmt, tile, y, sinv, y_t, sinv_t, s);
}

}  // namespace fp8lin
