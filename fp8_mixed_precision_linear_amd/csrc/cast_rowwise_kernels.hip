// cast_rowwise_kernels.hip -- row-wise (per-channel) FP8 quantisation on gfx950.
//
// [MPG] = "Mixed Precision LLM Training: The Complete Guide", "Per-row vs
//   per-tensor scaling": one scale per row instead of one per tensor, so an
//   outlier row or column only sets its own scale.
//
//   y   [rows][cols]: row r quantised with s_r = fl32(fmax / max_c |x[r][c]|)
//       (1 for an all-zero or non-finite row), scale_inv[r] = fl32(1 / s_r);
//   y_t [cols][rows]: row c of y_t (column c of x) quantised with the
//       column's own scale from max_r |x[r][c]|, scale_inv_t[c] -- the
//       operand of the GEMMs that reduce over rows (weight gradient).
// Codes as in the per-tensor cast (saturating RNE, NaN -> 0x7F | sign).
//
// Fast path (cols % 8 == 0 and cols <= 32768; with y_t also rows >= 64,
// rows % 16 == 0 and cols % 16 == 0), HBM-bound, x read twice when y_t is
// wanted:
//   1. row kernel: each group of NT threads owns whole rows (G groups per
//      workgroup, a persistent grid walks the rows), holds a row in
//      registers (8 bf16 per thread per chunk of 8*NT columns): row amax,
//      scale, cast, 8-byte stores.  Each thread keeps running maxima of its
//      columns over the rows it visits; at the end they are combined across
//      the groups in LDS and stored as the workgroup's partial column maxima
//      (16-bit |bf16| patterns, one row of [grid][cols]) in the memory of
//      y_t, which is written only later (grid <= rows / 2, so they fit);
//   2. the partial maxima are reduced per column into scale_inv_t (binary32
//      patterns of the column amax) -- no device atomics anywhere;
//   3. cast + transpose with per-column scales: 128 x 128 tiles through LDS
//      (the per-tensor kernel's layout), scales from the column maxima;
//   4. the column maxima become scale_inv_t in place.
// Other shapes: a workgroup per row, then a thread per column, element by
// element (same arithmetic).
#include "fp8_device.h"
#include "launch.h"

namespace fp8lin {

namespace {

// Scale of a row or column from its amax pattern (1 for zero / non-finite).
template <int FMT>
__device__ __forceinline__ void rw_scale(uint32_t amax_bits, float& s, float& si) {
  s = 1.0f;
  si = 1.0f;
  scale_from_amax(__uint_as_float(amax_bits), Fmt<FMT>::max, 0, s, si);
}

__device__ __forceinline__ void st_nt8(uint2 v, void* p) {
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  u32x2_t w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(p));
}

// ---------------------------------------------------------------------
// Row kernel.  Group g of workgroup b handles rows (b*G + g) + k*G*grid;
// thread t of a group holds columns c*8*NT + 8t .. +7 for c < NCH.  The
// trip count is the same for every group, so the per-row barrier is
// uniform; the row-amax slots are double-buffered (one barrier per row).
// ---------------------------------------------------------------------
template <int FMT, int NT, int G, int NCH, bool WANT_Y, bool COLS>
__global__ void __launch_bounds__(NT * G)
    k_rw_rows(const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t iters,
              uint8_t* __restrict__ y, float* __restrict__ sinv, uint32_t* __restrict__ part) {
  constexpr int NW = NT / 64;
  constexpr int CH = 8 * NT;
  __shared__ uint32_t red[2][G][NW];
  const int grp = threadIdx.x / NT, t = threadIdx.x % NT;
  const int lane = t & 63, wave = t >> 6;
  uint32_t cm[NCH][4];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int k = 0; k < 4; ++k) cm[c][k] = 0u;

  for (int64_t it = 0; it < iters; ++it) {
    const int64_t r = (it * gridDim.x + blockIdx.x) * G + grp;
    const bool have = r < rows;
    const uint16_t* xr = x + (have ? r : 0) * cols;
    uint4 v[NCH];
    uint32_t m = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int64_t col = (int64_t)c * CH + 8 * t;
      v[c] = make_uint4(0, 0, 0, 0);
      // cols % 8 == 0: all 8 in or out.  An ordinary load: the transposed
      // pass reads x again, from the last-level cache when it stayed there
      if (have && col < cols) v[c] = *reinterpret_cast<const uint4*>(xr + col);
      m = absmax_pk(m, v[c].x); m = absmax_pk(m, v[c].y);
      m = absmax_pk(m, v[c].z); m = absmax_pk(m, v[c].w);
      if constexpr (COLS) {
        cm[c][0] = absmax_pk(cm[c][0], v[c].x); cm[c][1] = absmax_pk(cm[c][1], v[c].y);
        cm[c][2] = absmax_pk(cm[c][2], v[c].z); cm[c][3] = absmax_pk(cm[c][3], v[c].w);
      }
    }
    if constexpr (WANT_Y) {
      const int par = (int)(it & 1);
      const uint32_t wm = wave_max_u32(absmax_fold(m));
      if (lane == 0) red[par][grp][wave] = wm;
      __syncthreads();
      uint32_t am = red[par][grp][0];
#pragma unroll
      for (int w = 1; w < NW; ++w) am = am > red[par][grp][w] ? am : red[par][grp][w];
      float s, si;
      rw_scale<FMT>(am, s, si);
      if (have) {
        if (t == 0) sinv[r] = si;
        uint8_t* yr = y + r * cols;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const int64_t col = (int64_t)c * CH + 8 * t;
          if (col < cols) st_nt8(cvt8_bf16<FMT>(v[c], s), yr + col);
        }
      }
    }
  }

  if constexpr (COLS) {
    // combine the groups' column maxima in LDS, one chunk at a time; the
    // workgroup's row of partials: packed pairs, part[blockIdx.x][cols / 2]
    __shared__ uint32_t cmx[G][4 * NT];
    uint32_t* prow = part + (int64_t)blockIdx.x * (cols >> 1);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if ((int64_t)c * CH >= cols) break;   // uniform
      __syncthreads();
#pragma unroll
      for (int k = 0; k < 4; ++k) cmx[grp][4 * t + k] = cm[c][k];
      __syncthreads();
      for (int d = threadIdx.x; d < 4 * NT; d += NT * G) {
        uint32_t pk = cmx[0][d];
#pragma unroll
        for (int g2 = 1; g2 < G; ++g2) pk = absmax_pk(pk, cmx[g2][d]);
        const int64_t col = (int64_t)c * CH + 2 * d;
        if (col < cols) prow[col >> 1] = pk;
      }
    }
  }
}

// ---------------------------------------------------------------------
// Cast + transpose with per-column scales.  rows % 16 == 0, cols % 16 ==
// 0.  Four 256-thread groups per workgroup, one 128 x 128 tile each per
// pass; thread t owns rows 4*(t/8)..+3 and columns 16*(t%8)..+15 of its
// tile.  The tile's 128 column scales are computed once into LDS.
// ---------------------------------------------------------------------
template <int FMT>
__global__ void __launch_bounds__(1024)
    k_rw_transpose(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                   const float* __restrict__ colmax, uint8_t* __restrict__ yt, int tiles_c,
                   int ntiles) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_all[4][128 * 128];
  __shared__ float scl[4][128];
  const int grp = threadIdx.x >> 8, t = threadIdx.x & 255;
  uint8_t* lds = lds_all[grp];
  const int cg = t & 7, rg = t >> 3;
  const int per_pass = (int)gridDim.x * 4;
  const int passes = (ntiles + per_pass - 1) / per_pass;   // uniform over the grid
  for (int ps = 0; ps < passes; ++ps) {
    const int tile = ps * per_pass + (int)blockIdx.x * 4 + grp;
    const bool have = tile < ntiles;
    const int64_t r0 = have ? (int64_t)(tile / tiles_c) * 128 : rows;
    const int64_t c0 = have ? (int64_t)(tile % tiles_c) * 128 : cols;
    const int64_t cbase = c0 + 16 * cg;
    const bool col_ok = cbase < cols;
    uint4 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = r0 + 4 * rg + i;
      a[i] = make_uint4(0, 0, 0, 0);
      b[i] = make_uint4(0, 0, 0, 0);
      if (col_ok && r < rows) {
        const uint4* p = reinterpret_cast<const uint4*>(x + r * cols + cbase);
        a[i] = ld_nt16(p);
        b[i] = ld_nt16(p + 1);
      }
    }
    if (t < 128) {
      float s, si;
      const int64_t c = c0 + t;
      rw_scale<FMT>(c < cols ? __float_as_uint(colmax[c]) : 0u, s, si);
      scl[grp][t] = s;
    }
    __syncthreads();
    float cs[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) cs[e] = scl[grp][16 * cg + e];
    uint32_t w[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 u = a[i], q = b[i];
      w[i][0] = cvt4<FMT>(bf16_lo(u.x) * cs[0], bf16_hi(u.x) * cs[1], bf16_lo(u.y) * cs[2],
                          bf16_hi(u.y) * cs[3]);
      w[i][1] = cvt4<FMT>(bf16_lo(u.z) * cs[4], bf16_hi(u.z) * cs[5], bf16_lo(u.w) * cs[6],
                          bf16_hi(u.w) * cs[7]);
      w[i][2] = cvt4<FMT>(bf16_lo(q.x) * cs[8], bf16_hi(q.x) * cs[9], bf16_lo(q.y) * cs[10],
                          bf16_hi(q.y) * cs[11]);
      w[i][3] = cvt4<FMT>(bf16_lo(q.z) * cs[12], bf16_hi(q.z) * cs[13], bf16_lo(q.w) * cs[14],
                          bf16_hi(q.w) * cs[15]);
    }
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
      const int idx = it * 256 + t;
      const int c = idx >> 3, ch = idx & 7;
      const int phys = ch ^ ((c >> 4) & 7);
      const int64_t gc = c0 + c, gr = r0 + 16 * ch;
      if (gc < cols && gr < rows) {
        const uint4 v = *reinterpret_cast<const uint4*>(lds + c * 128 + phys * 16);
        st_out16(v, yt + gc * rows + gr);
      }
    }
    __syncthreads();   // the next pass overwrites the tile and its scales
  }
}

// Partial column maxima [nparts][cols / 2] (packed pairs) -> binary32
// patterns of the column amax in colmax.  Block (16 pairs: 64 contiguous
// bytes per partial row) x (64 slices of the partial rows), combined in
// LDS: many small blocks, so the reads are spread over the whole chip.
__global__ void __launch_bounds__(1024)
    k_rw_colmax(const uint32_t* __restrict__ part, int64_t nparts, int64_t cols,
                float* __restrict__ colmax) {
  __shared__ uint32_t red[64][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t pairs = cols >> 1;
  const int64_t pr = (int64_t)blockIdx.x * 16 + tx;
  uint32_t m = 0;
  if (pr < pairs)
    for (int64_t b = ty; b < nparts; b += 64) m = absmax_pk(m, part[b * pairs + pr]);
  red[ty][tx] = m;
  __syncthreads();
  if (ty == 0 && pr < pairs) {
    for (int k = 1; k < 64; ++k) m = absmax_pk(m, red[k][tx]);
    colmax[2 * pr] = __uint_as_float((m & 0xFFFFu) << 16);
    colmax[2 * pr + 1] = __uint_as_float(m & 0xFFFF0000u);
  }
}

// Column maxima -> scale_inv_t, in place.
template <int FMT>
__global__ void k_rw_finalize(float* __restrict__ colmax, int64_t cols) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= cols) return;
  float s, si;
  rw_scale<FMT>(__float_as_uint(colmax[c]), s, si);
  colmax[c] = si;
}

// ---------------------------------------------------------------------
// Generic path.  Rows: one 256-thread workgroup per row (grid-stride),
// amax then cast.  Columns: one thread per column (grid-stride), amax then
// cast into the column's y_t row.
// ---------------------------------------------------------------------
template <int FMT>
__global__ void __launch_bounds__(256)
    k_rw_rows_generic(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                      uint8_t* __restrict__ y, float* __restrict__ sinv) {
  __shared__ uint32_t red[4];
  const int t = threadIdx.x;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const uint16_t* xr = x + r * cols;
    uint32_t m = 0;
    for (int64_t c = t; c < cols; c += 256) {
      const uint32_t b = (uint32_t)(xr[c] & 0x7FFFu) << 16;
      m = m > b ? m : b;
    }
    m = wave_max_u32(m);
    __syncthreads();   // the previous row's readers are done with red
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    uint32_t am = red[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) am = am > red[w] ? am : red[w];
    float s, si;
    rw_scale<FMT>(am, s, si);
    if (t == 0) sinv[r] = si;
    for (int64_t c = t; c < cols; c += 256)
      y[r * cols + c] =
          (uint8_t)(cvt4<FMT>(__uint_as_float((uint32_t)xr[c] << 16) * s, 0.f, 0.f, 0.f) & 0xFFu);
  }
}

template <int FMT>
__global__ void __launch_bounds__(256)
    k_rw_cols_generic(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                      uint8_t* __restrict__ yt, float* __restrict__ sinv_t) {
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < cols;
       c += (int64_t)gridDim.x * blockDim.x) {
    uint32_t m = 0;
    for (int64_t r = 0; r < rows; ++r) {
      const uint32_t b = (uint32_t)(x[r * cols + c] & 0x7FFFu) << 16;
      m = m > b ? m : b;
    }
    float s, si;
    rw_scale<FMT>(m, s, si);
    sinv_t[c] = si;
    for (int64_t r = 0; r < rows; ++r)
      yt[c * rows + r] = (uint8_t)(
          cvt4<FMT>(__uint_as_float((uint32_t)x[r * cols + c] << 16) * s, 0.f, 0.f, 0.f) & 0xFFu);
  }
}

// Launches the row kernel; with part != nullptr the workgroups' partial
// column maxima go to part ([grid][cols / 2] dwords, grid <= rows / 2 so
// that they fit in y_t's rows * cols bytes).  Returns the grid in *grid_out.
template <int FMT, int NT, int G, int NCH>
hipError_t launch_rows(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* y, float* sinv,
                       uint32_t* part, int per_cu, int64_t* grid_out, hipStream_t s) {
  const int64_t groups = (rows + G - 1) / G;
  int64_t grid = device_cu_count() * per_cu;
  if (grid > groups) grid = groups;
  if (part && grid > rows / 2) grid = rows / 2;
  if (grid < 1) grid = 1;
  *grid_out = grid;
  const int64_t iters = (groups + grid - 1) / grid;
  dim3 g((unsigned)grid), b(NT * G);
  if (y && part)
    hipLaunchKernelGGL((k_rw_rows<FMT, NT, G, NCH, true, true>), g, b, 0, s, x, rows, cols, iters,
                       y, sinv, part);
  else if (y)
    hipLaunchKernelGGL((k_rw_rows<FMT, NT, G, NCH, true, false>), g, b, 0, s, x, rows, cols, iters,
                       y, sinv, part);
  else
    hipLaunchKernelGGL((k_rw_rows<FMT, NT, G, NCH, false, true>), g, b, 0, s, x, rows, cols, iters,
                       y, sinv, part);
  return hipGetLastError();
}

// Row kernel for one of the row lengths <= 4096, 8192, 16384, 32768
// columns (8 * NT * NCH); part as in launch_rows.
template <int FMT>
hipError_t launch_rows_any(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* y, float* sinv,
                           uint32_t* part, int64_t* grid, hipStream_t s) {
  if (cols <= 4096) return launch_rows<FMT, 256, 4, 2>(x, rows, cols, y, sinv, part, 2, grid, s);
  if (cols <= 8192) return launch_rows<FMT, 256, 4, 4>(x, rows, cols, y, sinv, part, 1, grid, s);
  if (cols <= 16384) return launch_rows<FMT, 256, 2, 8>(x, rows, cols, y, sinv, part, 1, grid, s);
  return launch_rows<FMT, 512, 1, 8>(x, rows, cols, y, sinv, part, 1, grid, s);
}

template <int FMT>
hipError_t launch_rw(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* y, float* sinv,
                     uint8_t* yt, float* sinv_t, hipStream_t s) {
  const int64_t cus = device_cu_count();
  const bool fast_rows = cols % 8 == 0 && cols <= 32768;
  const bool fast_t = rows >= 64 && rows % 16 == 0 && cols % 16 == 0 &&
                      (rows + 127) / 128 * ((cols + 127) / 128) < (1LL << 30);
  hipError_t e = hipSuccess;
  int64_t grid = 0;
  if (!yt || !(fast_rows && fast_t)) {
    if (y && fast_rows) {
      e = launch_rows_any<FMT>(x, rows, cols, y, sinv, nullptr, &grid, s);
    } else if (y) {
      grid = rows < cus * 8 ? rows : cus * 8;
      hipLaunchKernelGGL((k_rw_rows_generic<FMT>), dim3((unsigned)grid), dim3(256), 0, s, x, rows,
                         cols, y, sinv);
      e = hipGetLastError();
    }
    if (e != hipSuccess || !yt) return e;
    grid = (cols + 255) / 256;
    if (grid > cus * 8) grid = cus * 8;
    hipLaunchKernelGGL((k_rw_cols_generic<FMT>), dim3((unsigned)grid), dim3(256), 0, s, x, rows,
                       cols, yt, sinv_t);
    return hipGetLastError();
  }
  // y_t wanted on the fast path: partial column maxima in y_t's memory
  uint32_t* part = reinterpret_cast<uint32_t*>(yt);
  e = launch_rows_any<FMT>(x, rows, cols, y, sinv, part, &grid, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_rw_colmax, dim3((unsigned)((cols / 2 + 15) / 16)), dim3(1024), 0, s, part,
                     grid, cols, sinv_t);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int tiles_c = (int)((cols + 127) / 128);
  const int ntiles = (int)((rows + 127) / 128) * tiles_c;
  int64_t blocks = (ntiles + 3) / 4;
  if (blocks > cus) blocks = cus;
  hipLaunchKernelGGL((k_rw_transpose<FMT>), dim3((unsigned)blocks), dim3(1024), 0, s, x, rows,
                     cols, sinv_t, yt, tiles_c, ntiles);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_rw_finalize<FMT>), dim3((unsigned)((cols + 255) / 256)), dim3(256), 0, s,
                     sinv_t, cols);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cast_rowwise(const uint16_t* x, int64_t rows, int64_t cols, int fmt, uint8_t* y,
                               float* sinv, uint8_t* y_t, float* sinv_t, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  return fmt == 0 ? launch_rw<0>(x, rows, cols, y, sinv, y_t, sinv_t, s)
                  : launch_rw<1>(x, rows, cols, y, sinv, y_t, sinv_t, s);
}

}  // namespace fp8lin
