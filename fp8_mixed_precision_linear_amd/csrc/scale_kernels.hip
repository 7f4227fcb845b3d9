// scale_kernels.hip -- amax reduction, scale computation and amax-history
// update for gfx950.
//
// [MPG] = "Mixed Precision LLM Training: The Complete Guide":
//   "Transformer Engine internals > Per-tensor scaling" (amax -> scale),
//   "Delayed scaling (the default recipe)", "History-based scaling",
//   "Calibration deep dive > Dynamic calibration (delayed scaling)".
#include <atomic>

#include "fp8_device.h"
#include "launch.h"

namespace fp8lin {

namespace {

constexpr int kAmaxThreads = 1024;

__global__ void k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = v;
}

// Block-wide max of one value per thread, then one device atomic per block.
__device__ __forceinline__ void block_max_to(float* out, uint32_t v) {
  __shared__ uint32_t part[kAmaxThreads / 64];
  v = wave_max_u32(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) part[wave] = v;
  __syncthreads();
  if (wave == 0) {
    uint32_t w = lane < (int)(blockDim.x >> 6) ? part[lane] : 0u;
    w = wave_max_u32(w);
    if (lane == 0 && w != 0u) atomic_max_bits(out, w);
  }
}

// max |x| over n bf16 values: 16-byte loads (8 values) on a grid-stride
// loop with up to kAmaxUnroll loads in flight per thread (issued together,
// then reduced), packed 16-bit max, then a wavefront / block reduction and one
// atomic per block.  With 2 loads per round trip the 4096 x 4096 case took
// four dependent trips through memory; with 8 a grid of one workgroup per
// CU covers it in one.
constexpr int kAmaxUnroll = 8;
__global__ void __launch_bounds__(kAmaxThreads) k_amax(const uint16_t* __restrict__ x, int64_t n,
                                                       float* __restrict__ amax) {
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const int64_t nv = n >> 3;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t mu[4] = {0u, 0u, 0u, 0u};
  for (; i < nv; i += kAmaxUnroll * stride) {
    uint4 v[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u)
      v[u] = i + u * stride < nv ? ld_nt16(xv + i + u * stride) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      uint32_t& m = mu[u & 3];
      m = absmax_pk(m, v[u].x); m = absmax_pk(m, v[u].y);
      m = absmax_pk(m, v[u].z); m = absmax_pk(m, v[u].w);
    }
  }
  uint32_t m = absmax_fold(absmax_pk(absmax_pk(mu[0], mu[1]), absmax_pk(mu[2], mu[3])));
  // tail: the last n % 8 values
  if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
    uint32_t t = (uint32_t)(x[(nv << 3) + threadIdx.x] & 0x7FFFu) << 16;
    m = m > t ? m : t;
  }
  block_max_to(amax, m);
}

// Saturation and underflow counts of the per-tensor cast, the overflow /
// underflow ratios of the diagnostic dashboard ([MPG] "Numerical-failure
// taxonomy > A diagnostic dashboard").  With v = fl32(x * s) as the cast
// computes it, an element saturates when |v| > the format's largest finite
// value (Inf included, NaN not) and underflows when x != 0 and |v| <= half
// the smallest subnormal step (2^-10 for E4M3, 2^-17 for E5M2): the RNE
// encode of such a value is +-0, the tie at exactly half a step going to
// the even code 0.  Both tests on the binary32 bit pattern of |v|.  Counts
// per thread, a block sum, and two 64-bit atomics per block into counts[].
template <int FMT>
__global__ void __launch_bounds__(kAmaxThreads) k_cast_stats(const uint16_t* __restrict__ x, int64_t n,
                                                             const float* __restrict__ scale,
                                                             unsigned long long* __restrict__ counts) {
  constexpr uint32_t kMaxBits = FMT == 0 ? 0x43E00000u : 0x47600000u;    // 448, 57344
  constexpr uint32_t kUnderBits = FMT == 0 ? 0x3A800000u : 0x37000000u;  // 2^-10, 2^-17
  const float s = *scale;
  uint32_t sat = 0, und = 0;
  auto one = [&](uint32_t h) {
    const uint32_t a = __float_as_uint(__uint_as_float(h << 16) * s) & 0x7FFFFFFFu;
    sat += (uint32_t)((a > kMaxBits) & (a <= 0x7F800000u));
    und += (uint32_t)(((h & 0x7FFFu) != 0u) & (a <= kUnderBits));
  };
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const int64_t nv = n >> 3;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nv; i += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = i + u * stride < nv ? ld_nt16(xv + i + u * stride) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) { one(w[k] & 0xFFFFu); one(w[k] >> 16); }
    }
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 7)) one(x[(nv << 3) + threadIdx.x]);
  // block sums (zero inputs -- padded loads and +0 -- count nowhere)
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    sat += __shfl_xor(sat, off, 64);
    und += __shfl_xor(und, off, 64);
  }
  __shared__ uint32_t part[2][kAmaxThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { part[0][wave] = sat; part[1][wave] = und; }
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long a = 0, b = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) { a += part[0][w]; b += part[1][w]; }
    if (a) atomicAdd(&counts[0], a);
    if (b) atomicAdd(&counts[1], b);
  }
}

// Current scaling: one thread per tensor.
__global__ void k_compute_scale(const float* __restrict__ amax, int64_t n, float fmax, int margin,
                                int pow2, float* __restrict__ scale,
                                float* __restrict__ scale_inv) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = 1.0f, si = 1.0f;
  if (pow2) pow2_scale_from_amax(amax[i], fmax, margin, s, si);
  else scale_from_amax(amax[i], fmax, margin, s, si);
  scale[i] = s;
  scale_inv[i] = si;
}

// Delayed scaling with an exponentially weighted amax ([MPG] "Delayed
// scaling (the default recipe)": an exponentially weighted average of
// recent steps), one thread per tensor.  A zero or non-finite new amax
// changes nothing; the first one seeds the average; afterwards
// ewma = fl32(fl32(beta * ewma) + fl32(fl32(1 - beta) * amax)), every
// operation rounded on its own (no contraction); the scale follows by the
// current-scaling rule and is kept when that rule fails.
__global__ void k_ewma_update(float* __restrict__ ewma, int64_t n, const float* __restrict__ amax_new,
                              float beta, float fmax, int margin, float* __restrict__ scale,
                              float* __restrict__ scale_inv) {
#pragma clang fp contract(off)
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float a = amax_new[i];
  if (!(a > 0.0f) || __builtin_isinf(a)) return;
  float e = ewma[i];
  if (e == 0.0f) {
    e = a;
  } else {
    const float t0 = beta * e;             // no fused multiply-add: each product
    const float t1 = (1.0f - beta) * a;    // and the sum round on their own
    e = t0 + t1;
  }
  ewma[i] = e;
  float sc, si;
  if (scale_from_amax(e, fmax, margin, sc, si)) {
    scale[i] = sc;
    scale_inv[i] = si;
  }
}

// Delayed scaling: one wavefront per tensor shifts its history (newest
// first), inserts the new amax, takes the window maximum (NaN propagates:
// compared as bit patterns of non-negative values) or the newest entry, and
// updates the scale only for a positive finite effective amax.  The shift
// runs over 64-entry chunks from the end backwards.  Within a chunk the one
// store instruction consumes the value of the one load instruction, so all
// lanes have read their source entries before any lane writes; the next
// (lower) chunk reads only entries below the ones already written.
//
// reset != 0: the consumed amax_new[i] is set to 0 afterwards (by lane 0,
// after every lane's read of it has returned: the value feeds the
// wavefront's reduction before the store is issued), ready for the next
// step's casts to max-accumulate into.
__global__ void __launch_bounds__(64) k_history_update(float* __restrict__ history, int64_t n,
                                                       int64_t len, float* amax_new,
                                                       float fmax, int margin, int algo, int pow2,
                                                       int reset, float* __restrict__ scale,
                                                       float* __restrict__ scale_inv) {
  const int64_t i = blockIdx.x;
  const int lane = threadIdx.x;
  float* h = history + i * len;
  const float a = amax_new[i];
  uint32_t best = __float_as_uint(a);
  for (int64_t base = ((len - 1) >> 6) << 6; base >= 0; base -= 64) {
    const int64_t j = base + lane;
    const bool have = j >= 1 && j < len;
    float v = 0.0f;
    if (have) v = h[j - 1];
    if (have) {
      h[j] = v;
      const uint32_t b = __float_as_uint(v);
      best = b > best ? b : best;
    }
  }
  best = wave_max_u32(best);
  if (lane == 0) {
    h[0] = a;
    const float eff = algo == 1 ? a : __uint_as_float(best);
    float s, si;
    const bool ok = pow2 ? pow2_scale_from_amax(eff, fmax, margin, s, si)
                         : scale_from_amax(eff, fmax, margin, s, si);
    if (ok) {
      scale[i] = s;
      scale_inv[i] = si;
    }
    if (reset) amax_new[i] = 0.0f;
  }
}

inline float fmax_of(int fmt) { return fmt == 0 ? kMaxE4M3 : kMaxE5M2; }

// max |x| over a [rows][cols] bf16 matrix with row stride ld (elements): a
// persistent grid walks the rows; 16-byte loads when every row start is
// 16-byte aligned (ld % 8 == 0), element loads otherwise and for the last
// cols % 8 values of a row.
__global__ void __launch_bounds__(kAmaxThreads) k_amax_rows(const uint16_t* __restrict__ x,
                                                            int64_t rows, int64_t cols, int64_t ld,
                                                            float* __restrict__ amax) {
  uint32_t mp = 0, m = 0;
  const bool vec = (ld & 7) == 0;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const uint16_t* xr = x + r * ld;
    int64_t c0 = 0;
    if (vec) {
      const int64_t nv = cols >> 3;
      for (int64_t i = threadIdx.x; i < nv; i += blockDim.x) {
        const uint4 a = ld_nt16(xr + 8 * i);
        mp = absmax_pk(mp, a.x); mp = absmax_pk(mp, a.y);
        mp = absmax_pk(mp, a.z); mp = absmax_pk(mp, a.w);
      }
      c0 = nv << 3;
    }
    for (int64_t c = c0 + threadIdx.x; c < cols; c += blockDim.x) {
      const uint32_t t = (uint32_t)(xr[c] & 0x7FFFu) << 16;
      m = m > t ? m : t;
    }
  }
  const uint32_t f = absmax_fold(mp);
  block_max_to(amax, m > f ? m : f);
}


}  // namespace

int64_t device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    v = 256;
  if (dev < 64) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_amax_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float* amax,
                            int acc, hipStream_t s) {
  hipError_t e = acc ? hipSuccess : launch_fill_u32(reinterpret_cast<uint32_t*>(amax), 1, 0u, s);
  if (e != hipSuccess || rows == 0 || cols == 0) return e;
  int64_t blocks = rows < device_cu_count() ? rows : device_cu_count();
  hipLaunchKernelGGL(k_amax_rows, dim3((unsigned)blocks), dim3(kAmaxThreads), 0, s, x, rows, cols,
                     ld, amax);
  return hipGetLastError();
}

hipError_t launch_amax(const uint16_t* x, int64_t n, float* amax, int acc, hipStream_t s) {
  hipError_t e = acc ? hipSuccess : launch_fill_u32(reinterpret_cast<uint32_t*>(amax), 1, 0u, s);
  if (e != hipSuccess || n == 0) return e;
  int64_t nv = n >> 3;
  // a persistent grid of at most one 1024-thread workgroup per CU: each
  // workgroup ends in one device atomic on the result, and those atomics
  // are serialised, so the grid is kept no larger than streaming needs.
  int64_t blocks = (nv + 2 * kAmaxThreads - 1) / (2 * kAmaxThreads);
  if (blocks < 1) blocks = 1;
  if (blocks > device_cu_count()) blocks = device_cu_count();
  hipLaunchKernelGGL(k_amax, dim3((unsigned)blocks), dim3(kAmaxThreads), 0, s, x, n, amax);
  return hipGetLastError();
}

hipError_t launch_cast_stats(const uint16_t* x, int64_t n, const float* scale, int fmt,
                             uint64_t* counts, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t nv = n >> 3;
  int64_t blocks = (nv + 4 * kAmaxThreads - 1) / (4 * kAmaxThreads);
  if (blocks < 1) blocks = 1;
  if (blocks > device_cu_count()) blocks = device_cu_count();
  auto c = reinterpret_cast<unsigned long long*>(counts);
  if (fmt == 0)
    hipLaunchKernelGGL(k_cast_stats<0>, dim3((unsigned)blocks), dim3(kAmaxThreads), 0, s, x, n, scale, c);
  else
    hipLaunchKernelGGL(k_cast_stats<1>, dim3((unsigned)blocks), dim3(kAmaxThreads), 0, s, x, n, scale, c);
  return hipGetLastError();
}

hipError_t launch_compute_scale(const float* amax, int64_t n, int fmt, int margin, int pow2,
                                float* scale, float* scale_inv, hipStream_t s) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_compute_scale, dim3((unsigned)blocks), dim3(256), 0, s, amax, n,
                     fmax_of(fmt), margin, pow2, scale, scale_inv);
  return hipGetLastError();
}

hipError_t launch_history_update(float* history, int64_t n, int64_t len, float* amax_new,
                                 int fmt, int margin, int algo, int pow2, int reset, float* scale,
                                 float* scale_inv, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (n > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_history_update, dim3((unsigned)n), dim3(64), 0, s, history, n, len,
                     amax_new, fmax_of(fmt), margin, algo, pow2, reset, scale, scale_inv);
  return hipGetLastError();
}

hipError_t launch_ewma_update(float* ewma, int64_t n, const float* amax_new, float beta, int fmt,
                              int margin, float* scale, float* scale_inv, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_ewma_update, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ewma, n,
                     amax_new, beta, fmax_of(fmt), margin, scale, scale_inv);
  return hipGetLastError();
}

}  // namespace fp8lin
