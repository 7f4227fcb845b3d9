// cast_kernels.hip -- per-tensor saturating RNE cast to FP8 on gfx950, with
// optional fused transpose (LDS-staged) and fused amax of the input.
//
// [MPG] = "Mixed Precision LLM Training: The Complete Guide",
//   "Transformer Engine internals > Per-tensor scaling": multiply by the
//   tensor's scale, then quantise.
// [TALK] = PyData Amsterdam 2026 "FP8 for pretraining", outline 05:00-15:00:
//   E4M3 for forward activations and weights, E5M2 for gradients.
//
// With SR the rounding is stochastic ([MPG] "Stochastic rounding"): each
// element draws its word of a Philox4x32-10 block (fp8_device.h) from its
// row-major index, the seed and the offset; the transposed copy holds the
// same codes.
//
// Memory-bound kernels: every byte is read or written once, with 16-byte
// accesses.  The transposed copy goes through LDS as dwords that each hold
// 4 codes of one column (a 4x4 byte transpose in registers), with a 16-byte
// XOR swizzle so that the writes and the 16-byte reads are conflict free.
#include "fp8_device.h"
#include "launch.h"

namespace fp8lin {

namespace {

constexpr int kThreads = 256;      // generic kernel
constexpr int kBig = 1024;         // persistent kernels: one workgroup per CU

// Workgroup maximum, then one device atomic per workgroup.  The casts with
// an amax run persistent grids of one workgroup per CU: device atomics on
// one address are serialised, so their number, not the data volume, sets
// the cost of the reduction.
template <int NT>
__device__ __forceinline__ void block_amax_to(float* out, uint32_t v) {
  __shared__ uint32_t part[NT / 64];
  v = wave_max_u32(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) part[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t w = part[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) w = w > part[i] ? w : part[i];
    if (w != 0u) atomic_max_bits(out, w);
  }
}

// ---------------------------------------------------------------------
// Flat cast (no transpose): 16 elements per thread per step (two 16-byte
// loads, one 16-byte store).  Any n; the last n % 16 values are handled by
// the first threads of block 0.
// ---------------------------------------------------------------------
template <int FMT, bool AMAX, bool SR>
__global__ void __launch_bounds__(kBig)
    k_cast_flat(const uint16_t* __restrict__ x, int64_t n, const float* __restrict__ scale,
                uint8_t* __restrict__ y, float* __restrict__ amax, uint64_t seed,
                uint64_t offset, const uint64_t* __restrict__ rng) {
  if constexpr (SR)
    if (rng) { seed = rng[0]; offset = rng[1]; }
  const float s = *scale;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint4* yv = reinterpret_cast<uint4*>(y);
  const int64_t nu = n >> 4;  // units of 16 elements
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t m = 0;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < nu; u += stride) {
    uint4 a = ld_nt16(xv + 2 * u);
    uint4 b = ld_nt16(xv + 2 * u + 1);
    if (AMAX) {
      m = absmax_pk(m, a.x); m = absmax_pk(m, a.y); m = absmax_pk(m, a.z); m = absmax_pk(m, a.w);
      m = absmax_pk(m, b.x); m = absmax_pk(m, b.y); m = absmax_pk(m, b.z); m = absmax_pk(m, b.w);
    }
    uint2 qa, qb;
    if constexpr (SR) {   // elements 16u .. 16u+15: blocks 4u .. 4u+3
      qa = cvt8_bf16_sr<FMT>(a, s, sr_block(4 * u, seed, offset), sr_block(4 * u + 1, seed, offset));
      qb = cvt8_bf16_sr<FMT>(b, s, sr_block(4 * u + 2, seed, offset),
                             sr_block(4 * u + 3, seed, offset));
    } else {
      qa = cvt8_bf16<FMT>(a, s);
      qb = cvt8_bf16<FMT>(b, s);
    }
    st_out16(make_uint4(qa.x, qa.y, qb.x, qb.y), yv + u);
  }
  uint32_t mb = AMAX ? absmax_fold(m) : 0u;
  if (blockIdx.x == 0 && threadIdx.x < (n & 15)) {
    int64_t i = (nu << 4) + threadIdx.x;
    uint16_t h = x[i];
    float v = __uint_as_float((uint32_t)h << 16) * s;
    if constexpr (SR) v = sr_target<FMT>(v, sr_word(i, seed, offset));
    y[i] = (uint8_t)(cvt4<FMT>(v, 0.f, 0.f, 0.f) & 0xFFu);
    if (AMAX) {
      uint32_t t = (uint32_t)(h & 0x7FFFu) << 16;
      mb = mb > t ? mb : t;
    }
  }
  if (AMAX) block_amax_to<kBig>(amax, mb);
}

// ---------------------------------------------------------------------
// Cast + transpose, tile 128 x 128, 256 threads.  Requires rows % 16 == 0
// and cols % 16 == 0 (16-byte rows in both orientations); tiles at the
// right / bottom edge may be partial in steps of 16.
// Thread t owns rows 4*(t/8) .. +3 and columns 16*(t%8) .. +15 of the tile.
// LDS holds the transposed tile: line c (a column of x, 128 bytes = 8
// chunks of 16 rows); chunk ch of line c sits at physical chunk
// ch ^ ((c/16) & 7).
// ---------------------------------------------------------------------
template <int FMT, bool AMAX, bool WANT_Y, bool SR>
__global__ void __launch_bounds__(kBig)
    k_cast_transpose(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                     const float* __restrict__ scale, uint8_t* __restrict__ y,
                     uint8_t* __restrict__ yt, float* __restrict__ amax, int tiles_c,
                     int ntiles, uint64_t seed, uint64_t offset,
                     const uint64_t* __restrict__ rng) {
  if constexpr (SR)
    if (rng) { seed = rng[0]; offset = rng[1]; }
  // four 256-thread groups, each on its own tile and 16 KB of LDS; the grid
  // walks the tiles row-major, four per workgroup per pass
  __shared__ __attribute__((aligned(16))) uint8_t lds_all[4][128 * 128];
  const float s = *scale;
  const int grp = threadIdx.x >> 8, t = threadIdx.x & 255;
  uint8_t* lds = lds_all[grp];
  const int cg = t & 7, rg = t >> 3;
  const int per_pass = (int)gridDim.x * 4;
  const int passes = (ntiles + per_pass - 1) / per_pass;   // uniform over the grid
  uint32_t m = 0;
  for (int ps = 0; ps < passes; ++ps) {
    const int tile = ps * per_pass + (int)blockIdx.x * 4 + grp;
    const bool have = tile < ntiles;
    const int64_t r0 = have ? (int64_t)(tile / tiles_c) * 128 : rows;
    const int64_t c0 = have ? (int64_t)(tile % tiles_c) * 128 : cols;
    const int64_t cbase = c0 + 16 * cg;
    const bool col_ok = cbase < cols;  // cols % 16 == 0: whole 16-col group in or out
    uint32_t w[4][4];                  // [row i][dword j]: codes of cols 4j..4j+3
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = r0 + 4 * rg + i;
      uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
      if (col_ok && r < rows) {
        const uint4* p = reinterpret_cast<const uint4*>(x + r * cols + cbase);
        a = ld_nt16(p);
        b = ld_nt16(p + 1);
      }
      if (AMAX) {
        m = absmax_pk(m, a.x); m = absmax_pk(m, a.y); m = absmax_pk(m, a.z); m = absmax_pk(m, a.w);
        m = absmax_pk(m, b.x); m = absmax_pk(m, b.y); m = absmax_pk(m, b.z); m = absmax_pk(m, b.w);
      }
      uint2 qa, qb;
      if constexpr (SR) {   // 16 elements from r * cols + cbase (a multiple of 16)
        const uint64_t g = (uint64_t)(r * cols + cbase) >> 2;
        qa = cvt8_bf16_sr<FMT>(a, s, sr_block(g, seed, offset), sr_block(g + 1, seed, offset));
        qb = cvt8_bf16_sr<FMT>(b, s, sr_block(g + 2, seed, offset), sr_block(g + 3, seed, offset));
      } else {
        qa = cvt8_bf16<FMT>(a, s);
        qb = cvt8_bf16<FMT>(b, s);
      }
      w[i][0] = qa.x; w[i][1] = qa.y; w[i][2] = qb.x; w[i][3] = qb.y;
      if (WANT_Y && col_ok && r < rows)
        st_out16(make_uint4(qa.x, qa.y, qb.x, qb.y), reinterpret_cast<uint4*>(y + r * cols + cbase));
    }
    // transposed dwords into LDS: column c = 16*cg + 4*j + k, rows 4*rg..+3
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t t0, t1, t2, t3;
      transpose4x4(w[0][j], w[1][j], w[2][j], w[3][j], t0, t1, t2, t3);
      const uint32_t tv[4] = {t0, t1, t2, t3};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = 16 * cg + 4 * j + k;
        const int ch = rg >> 2, within = rg & 3;
        const int phys = ch ^ ((c >> 4) & 7);
        *reinterpret_cast<uint32_t*>(lds + c * 128 + phys * 16 + within * 4) = tv[k];
      }
    }
    __syncthreads();
    // y_t rows: tile column c -> y_t row c0 + c, 16 bytes = rows 16*ch..+15
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = it * 256 + t;  // 0..1023
      const int c = idx >> 3, ch = idx & 7;
      const int phys = ch ^ ((c >> 4) & 7);
      const int64_t gc = c0 + c, gr = r0 + 16 * ch;
      if (gc < cols && gr < rows) {
        uint4 v = *reinterpret_cast<const uint4*>(lds + c * 128 + phys * 16);
        st_out16(v, (yt + gc * rows + gr));
      }
    }
    __syncthreads();   // the next pass overwrites the LDS tile
  }
  if (AMAX) block_amax_to<kBig>(amax, absmax_fold(m));
}

// ---------------------------------------------------------------------
// Generic cast for shapes the tiled kernels do not take (rows or cols not
// multiples of 16): one element per thread, same arithmetic.
// ---------------------------------------------------------------------
template <int FMT, bool AMAX, bool SR>
__global__ void __launch_bounds__(kThreads)
    k_cast_generic(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                   const float* __restrict__ scale, uint8_t* __restrict__ y,
                   uint8_t* __restrict__ yt, float* __restrict__ amax, uint64_t seed,
                   uint64_t offset, const uint64_t* __restrict__ rng) {
  if constexpr (SR)
    if (rng) { seed = rng[0]; offset = rng[1]; }
  const float s = *scale;
  const int64_t n = rows * cols;
  uint32_t m = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint16_t h = x[i];
    float v = __uint_as_float((uint32_t)h << 16) * s;
    if constexpr (SR) v = sr_target<FMT>(v, sr_word(i, seed, offset));
    const uint8_t q = (uint8_t)(cvt4<FMT>(v, 0.f, 0.f, 0.f) & 0xFFu);
    const int64_t r = i / cols, c = i - r * cols;
    if (y) y[i] = q;
    if (yt) yt[c * rows + r] = q;
    if (AMAX) {
      uint32_t t = (uint32_t)(h & 0x7FFFu) << 16;
      m = m > t ? m : t;
    }
  }
  if (AMAX) block_amax_to<kThreads>(amax, m);
}

// The generator state of a stochastic-rounding cast that reads (seed,
// offset) from device memory moves on by `adv` once the cast has read it.
__global__ void k_rng_advance(uint64_t* rng, uint64_t adv) {
  if (threadIdx.x == 0 && blockIdx.x == 0) rng[1] += adv;
}

template <int FMT, bool AMAX, bool SR>
hipError_t launch_cast_t(const uint16_t* x, int64_t rows, int64_t cols, const float* scale,
                         uint8_t* y, uint8_t* yt, float* amax, uint64_t seed, uint64_t offset,
                         const uint64_t* rng, hipStream_t s) {
  const int64_t n = rows * cols;
  const int64_t cus = device_cu_count();
  if (yt == nullptr) {
    int64_t nu = n >> 4;
    int64_t blocks = (nu + kBig - 1) / kBig;
    if (blocks > cus) blocks = cus;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL((k_cast_flat<FMT, AMAX, SR>), dim3((unsigned)blocks), dim3(kBig), 0, s, x,
                       n, scale, y, amax, seed, offset, rng);
    return hipGetLastError();
  }
  if (rows % 16 == 0 && cols % 16 == 0 && (rows + 127) / 128 * ((cols + 127) / 128) < (1LL << 30)) {
    const int tiles_c = (int)((cols + 127) / 128);
    const int ntiles = (int)((rows + 127) / 128) * tiles_c;
    int64_t blocks = (ntiles + 3) / 4;
    if (blocks > cus) blocks = cus;
    if (y)
      hipLaunchKernelGGL((k_cast_transpose<FMT, AMAX, true, SR>), dim3((unsigned)blocks),
                         dim3(kBig), 0, s, x, rows, cols, scale, y, yt, amax, tiles_c, ntiles,
                         seed, offset, rng);
    else
      hipLaunchKernelGGL((k_cast_transpose<FMT, AMAX, false, SR>), dim3((unsigned)blocks),
                         dim3(kBig), 0, s, x, rows, cols, scale, y, yt, amax, tiles_c, ntiles,
                         seed, offset, rng);
    return hipGetLastError();
  }
  int64_t blocks = (n + kThreads - 1) / kThreads;
  if (blocks > cus) blocks = cus;
  hipLaunchKernelGGL((k_cast_generic<FMT, AMAX, SR>), dim3((unsigned)blocks), dim3(kThreads), 0, s,
                     x, rows, cols, scale, y, yt, amax, seed, offset, rng);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cast(const uint16_t* x, int64_t rows, int64_t cols, const float* scale, int fmt,
                       uint8_t* y, uint8_t* y_t, float* amax, int amax_acc, int sr, uint64_t seed,
                       uint64_t offset, uint64_t* rng, uint64_t advance, hipStream_t s) {
  if (amax && !amax_acc) {
    hipError_t e = launch_fill_u32(reinterpret_cast<uint32_t*>(amax), 1, 0u, s);
    if (e != hipSuccess) return e;
  }
  hipError_t e = hipSuccess;
  if (rows != 0 && cols != 0) {
    const int key = fmt * 4 + (amax ? 2 : 0) + (sr ? 1 : 0);
    const uint64_t* r = rng;
    switch (key) {
      case 0: e = launch_cast_t<0, false, false>(x, rows, cols, scale, y, y_t, amax, seed, offset, r, s); break;
      case 1: e = launch_cast_t<0, false, true>(x, rows, cols, scale, y, y_t, amax, seed, offset, r, s); break;
      case 2: e = launch_cast_t<0, true, false>(x, rows, cols, scale, y, y_t, amax, seed, offset, r, s); break;
      case 3: e = launch_cast_t<0, true, true>(x, rows, cols, scale, y, y_t, amax, seed, offset, r, s); break;
      case 4: e = launch_cast_t<1, false, false>(x, rows, cols, scale, y, y_t, amax, seed, offset, r, s); break;
      case 5: e = launch_cast_t<1, false, true>(x, rows, cols, scale, y, y_t, amax, seed, offset, r, s); break;
      case 6: e = launch_cast_t<1, true, false>(x, rows, cols, scale, y, y_t, amax, seed, offset, r, s); break;
      default: e = launch_cast_t<1, true, true>(x, rows, cols, scale, y, y_t, amax, seed, offset, r, s); break;
    }
    if (e != hipSuccess) return e;
  }
  if (rng && advance) {   // after the cast has read the state (stream order)
    hipLaunchKernelGGL(k_rng_advance, dim3(1), dim3(64), 0, s, rng, advance);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace fp8lin
