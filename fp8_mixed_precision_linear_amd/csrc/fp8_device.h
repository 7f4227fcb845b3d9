// fp8_device.h -- device-side helpers of the FP8 scaled linear layer (gfx950).
//
// FP8 codes are the OCP encodings that gfx950's conversion and matrix
// instructions use natively: E4M3 (max 448, no Inf) and E5M2 (max 57344).
// Sources, cited by page title and section:
//   [MPG] "Mixed Precision LLM Training: The Complete Guide":
//         "The precision formats", "FP8 E4M3", "FP8 E5M2",
//         "Transformer Engine internals > Per-tensor scaling".
//   [P3]  "Training and inference of large language models using 8-bit
//         floating point" (arXiv 2309.17224 library entry).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8lin {

constexpr float kMaxE4M3 = 448.0f;
constexpr float kMaxE5M2 = 57344.0f;
constexpr float kFltMax = 3.402823466e+38f;

template <int FMT>
struct Fmt;
template <>
struct Fmt<0> {
  static constexpr float max = kMaxE4M3;
};
template <>
struct Fmt<1> {
  static constexpr float max = kMaxE5M2;
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte streaming (non-temporal) global load / store.
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
  u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
// FP8 outputs of the casts: a GEMM reads them next, so they are written
// with ordinary stores, which leave them in the last-level cache (the
// 256 MB MALL holds every operand of a 4096^3 step) instead of streaming
// them past it as a non-temporal store does.
__device__ __forceinline__ void st_out16(uint4 v, void* p) { *reinterpret_cast<uint4*>(p) = v; }
__device__ __forceinline__ void st_nt16(uint4 v, void* p) {
  u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Saturation before the hardware conversion: finite values beyond the
// format's largest magnitude and +-Inf become +-max.  Values between max and
// the rounding midpoint above it round to max anyway, so clamping first and
// rounding second equals rounding first and saturating second.
template <int FMT>
__device__ __forceinline__ float sat(float v) {
  return __builtin_amdgcn_fmed3f(v, -Fmt<FMT>::max, Fmt<FMT>::max);
}

// The conversion instructions emit one fixed NaN code whatever the input's
// sign; the layer's cast maps NaN to 0x7F | sign.  Only wavefronts that
// actually hold a NaN take this path.  The out-of-line copy keeps the casts'
// loops small; the inlined one serves kernels whose register file is nearly
// full, where a call would spill the caller's live registers to scratch.
__device__ __forceinline__ uint32_t nan_patch_inl(uint32_t w, float a, float b, float c, float d) {
  const float v[4] = {a, b, c, d};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (__builtin_isnan(v[i])) {
      const uint32_t code = 0x7Fu | ((__float_as_uint(v[i]) >> 24) & 0x80u);
      w = (w & ~(0xFFu << (8 * i))) | (code << (8 * i));
    }
  return w;
}
__device__ __noinline__ uint32_t nan_patch(uint32_t w, float a, float b, float c, float d) {
  return nan_patch_inl(w, a, b, c, d);
}

// Four binary32 values -> four FP8 codes packed little-endian in a dword
// (a in byte 0 ... d in byte 3), round to nearest even, saturating.
template <int FMT, bool INLINE_NAN = false>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  int w;
  if constexpr (FMT == 0) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(sat<0>(a), sat<0>(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(sat<0>(c), sat<0>(d), w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(sat<1>(a), sat<1>(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(sat<1>(c), sat<1>(d), w, true);
  }
  if (__builtin_isnan(a) | __builtin_isnan(b) | __builtin_isnan(c) | __builtin_isnan(d))
    return INLINE_NAN ? nan_patch_inl((uint32_t)w, a, b, c, d) : nan_patch((uint32_t)w, a, b, c, d);
  return (uint32_t)w;
}

// Eight bf16 (one 16-byte load, as 4 dwords) times s -> 8 codes (2 dwords).
template <int FMT>
__device__ __forceinline__ uint2 cvt8_bf16(uint4 v, float s) {
  uint2 r;
  r.x = cvt4<FMT>(bf16_lo(v.x) * s, bf16_hi(v.x) * s, bf16_lo(v.y) * s, bf16_hi(v.y) * s);
  r.y = cvt4<FMT>(bf16_lo(v.z) * s, bf16_hi(v.z) * s, bf16_lo(v.w) * s, bf16_hi(v.w) * s);
  return r;
}

// ---------------------------------------------------------------------
// Stochastic rounding ([MPG] "Stochastic rounding": round up or down at
// random according to the remainder, so the rounded value is unbiased).
//
// Random words: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011).  Element i of a tensor (row-major
// index) takes word i % 4 of the block with counter (i / 4, offset) as four
// little-endian 32-bit words and key seed.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    // one 32x32 -> 64-bit multiply gives both halves
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x, p1 = (uint64_t)0xCD9E8D57u * c.z;
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// The four words of block g (elements 4g .. 4g+3).
__device__ __forceinline__ uint4 sr_block(uint64_t g, uint64_t seed, uint64_t offset) {
  return philox4x32_10(make_uint4((uint32_t)g, (uint32_t)(g >> 32), (uint32_t)offset,
                                  (uint32_t)(offset >> 32)),
                       (uint32_t)seed, (uint32_t)(seed >> 32));
}

// Word i % 4 of block i / 4 (one element on its own).
__device__ __forceinline__ uint32_t sr_word(int64_t i, uint64_t seed, uint64_t offset) {
  const uint4 w = sr_block((uint64_t)i >> 2, seed, offset);
  const int k = (int)(i & 3);
  return k == 0 ? w.x : (k == 1 ? w.y : (k == 2 ? w.z : w.w));
}

// The FP8 value (as an exactly representable binary32) that v rounds to
// with the word r: with lo <= |v| < hi the neighbouring FP8 magnitudes, hi
// when r < (|v| - lo) / (hi - lo) * 2^32, else lo; sign kept.  |v| >= fmax,
// Inf and NaN are returned as they are (the conversion saturates them and
// patches NaN).  In the FP8 normal range the remainder is the low 23 - M
// mantissa bits of |v|; below it (rare: a branch), |v| is scaled by the
// inverse subnormal step (exact), and r < F with F = remainder * 2^32 (an
// exact binary32 below 2^32) is decided as r < ceil(F) in 64-bit integers.
template <int FMT>
__device__ __noinline__ uint32_t sr_subnormal(float a, uint32_t r) {
  constexpr int MB = FMT == 0 ? 3 : 2;
  constexpr int EMIN = FMT == 0 ? -6 : -14;
  const float x = __builtin_ldexpf(a, MB - EMIN);            // a / subnormal step, exact
  const float k = __builtin_floorf(x);
  const float F = __builtin_ldexpf(x - k, 32);               // exact, < 2^32
  const bool up = (uint64_t)r < (uint64_t)__builtin_ceilf(F);
  return __float_as_uint(__builtin_ldexpf(k + (up ? 1.0f : 0.0f), EMIN - MB));
}

template <int FMT>
__device__ __forceinline__ float sr_target(float v, uint32_t r) {
  constexpr int MB = FMT == 0 ? 3 : 2;           // mantissa bits
  constexpr int EMIN = FMT == 0 ? -6 : -14;      // exponent of the smallest normal
  constexpr int D = 23 - MB;
  const float a = __builtin_fabsf(v);
  if (!(a < Fmt<FMT>::max)) return v;
  const uint32_t sgn = __float_as_uint(v) & 0x80000000u;
  const uint32_t b = __float_as_uint(a);
  uint32_t t;
  if (__builtin_expect(b >= (uint32_t)(EMIN + 127) << 23, 1)) {
    const uint32_t frac = b & ((1u << D) - 1u);
    const bool up = (r >> (32 - D)) < frac;
    t = (b & ~((1u << D) - 1u)) + (up ? (1u << D) : 0u);
  } else {
    t = sr_subnormal<FMT>(a, r);   // out of line: keeps the common path short
  }
  return __uint_as_float(t | sgn);
}

// Eight bf16 (one 16-byte load) times s -> 8 codes, stochastically rounded
// with the words w[0..7].
template <int FMT>
__device__ __forceinline__ uint2 cvt8_bf16_sr(uint4 v, float s, uint4 w0, uint4 w1) {
  uint2 q;
  q.x = cvt4<FMT>(sr_target<FMT>(bf16_lo(v.x) * s, w0.x), sr_target<FMT>(bf16_hi(v.x) * s, w0.y),
                  sr_target<FMT>(bf16_lo(v.y) * s, w0.z), sr_target<FMT>(bf16_hi(v.y) * s, w0.w));
  q.y = cvt4<FMT>(sr_target<FMT>(bf16_lo(v.z) * s, w1.x), sr_target<FMT>(bf16_hi(v.z) * s, w1.y),
                  sr_target<FMT>(bf16_lo(v.w) * s, w1.z), sr_target<FMT>(bf16_hi(v.w) * s, w1.w));
  return q;
}

// max |x| over the bf16 halves of a dword, as a packed pair of 15-bit
// magnitudes: clearing the sign bits leaves patterns whose unsigned order
// is the order of |x| (NaN above Inf), so a packed u16 max is exact.
__device__ __forceinline__ uint32_t absmax_pk(uint32_t acc, uint32_t w) {
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
  us2 a = __builtin_bit_cast(us2, acc);
  us2 b = __builtin_bit_cast(us2, w & 0x7FFF7FFFu);
  us2 m = __builtin_elementwise_max(a, b);
  return __builtin_bit_cast(uint32_t, m);
}

// Fold a packed pair into the binary32 bit pattern of the larger |x|.
__device__ __forceinline__ uint32_t absmax_fold(uint32_t pk) {
  uint32_t lo = pk & 0xFFFFu, hi = pk >> 16;
  return (lo > hi ? lo : hi) << 16;
}

// Maximum over the 64 lanes of a wavefront (unsigned).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

// Scale from an amax: s = fl32(fmax / amax) * 2^-margin, s_inv = fl32(1/s)
// (both divisions correctly rounded); returns false (and leaves s, s_inv
// untouched) for amax == 0 or non-finite.  A quotient that overflows
// binary32 is clamped to FLT_MAX.  [MPG] "Per-tensor scaling"; the recipe's
// `margin` read as a division by 2^margin.
__device__ __forceinline__ bool scale_from_amax(float amax, float fmax, int margin, float& s,
                                                float& s_inv) {
  if (!(amax > 0.0f) || __builtin_isinf(amax)) return false;   // also rejects NaN
  float q = __fdiv_rn(fmax, amax);
  if (__builtin_isinf(q)) q = kFltMax;
  if (margin != 0) q = __builtin_ldexpf(q, -margin);
  s = q;
  s_inv = __fdiv_rn(1.0f, q);
  return true;
}

// Power-of-two ("exponent bias") scale from an amax: s = 2^e with e the
// largest integer such that amax * 2^e <= fmax, minus margin, clamped to
// [-126, 126]; s_inv = 2^-e (both exact normal powers of two).  Returns
// false (s, s_inv untouched) for amax == 0 or non-finite.  With
// amax = 1.ma * 2^ea and fmax = 1.mf * 2^ef: e = ef - ea when ma <= mf,
// else ef - ea - 1 (compared on the mantissa fields; a subnormal amax is
// first scaled by 2^64, exactly).  [P3] "Training and inference of large
// language models using 8-bit floating point": the exponent bias is chosen
// from the tensor's maximum (FP8-AMAX).
__device__ __forceinline__ bool pow2_scale_from_amax(float amax, float fmax, int margin, float& s,
                                                     float& s_inv) {
  if (!(amax > 0.0f) || __builtin_isinf(amax)) return false;   // also rejects NaN
  int adj = 0;
  if (amax < 1.17549435e-38f) {
    amax *= 18446744073709551616.0f;   // 2^64
    adj = 64;
  }
  const uint32_t b = __float_as_uint(amax), f = __float_as_uint(fmax);
  const int ea = (int)(b >> 23) - 127 - adj, ef = (int)(f >> 23) - 127;
  int e = ef - ea - ((b & 0x7FFFFFu) > (f & 0x7FFFFFu) ? 1 : 0) - margin;
  e = e > 126 ? 126 : (e < -126 ? -126 : e);
  s = __uint_as_float((uint32_t)(e + 127) << 23);
  s_inv = __uint_as_float((uint32_t)(127 - e) << 23);
  return true;
}

// Device-scope atomic max on the bits of a non-negative binary32 value
// (unsigned order = value order for patterns with the sign bit clear).
// Device-scope atomics on one address are serialised where the XCDs meet
// (measured on gfx950: ~10 ns each, so a few thousand of them cost tens of
// microseconds), so the current value is read first and the atomic is
// issued only when it would raise it.  The stored value only grows, so a
// stale read costs at most a redundant atomic, never a lost maximum.
__device__ __forceinline__ void atomic_max_bits(float* dst, uint32_t bits) {
  unsigned int* p = reinterpret_cast<unsigned int*>(dst);
  const unsigned int cur = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (bits > cur) atomicMax(p, bits);
}

// ---------------------------------------------------------------------
// Helpers shared by the cast and GEMM kernels.

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// 4 x 4 byte transpose in registers: wK holds bytes [row K][col 0..3], tJ
// receives bytes [row 0..3][col J].  __builtin_amdgcn_perm(hi, lo, sel):
// selector bytes 0-3 pick from lo, 4-7 from hi.
__device__ __forceinline__ void transpose4x4(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                             uint32_t& t0, uint32_t& t1, uint32_t& t2,
                                             uint32_t& t3) {
  const uint32_t a01_lo = __builtin_amdgcn_perm(w1, w0, 0x05010400u);  // r0c0 r1c0 r0c1 r1c1
  const uint32_t a01_hi = __builtin_amdgcn_perm(w1, w0, 0x07030602u);  // r0c2 r1c2 r0c3 r1c3
  const uint32_t a23_lo = __builtin_amdgcn_perm(w3, w2, 0x05010400u);  // r2c0 r3c0 r2c1 r3c1
  const uint32_t a23_hi = __builtin_amdgcn_perm(w3, w2, 0x07030602u);  // r2c2 r3c2 r2c3 r3c3
  t0 = __builtin_amdgcn_perm(a23_lo, a01_lo, 0x05040100u);             // column 0
  t1 = __builtin_amdgcn_perm(a23_lo, a01_lo, 0x07060302u);             // column 1
  t2 = __builtin_amdgcn_perm(a23_hi, a01_hi, 0x05040100u);             // column 2
  t3 = __builtin_amdgcn_perm(a23_hi, a01_hi, 0x07060302u);             // column 3
}

// binary32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40u);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// One v_mfma_f32_16x16x128_f8f6f4: c + a . b with FP8 operands, format codes
// 0 = E4M3 (fp8), 1 = E5M2 (bf8) per operand; zero scale operands select the
// unscaled instruction.
template <int AF, int BF>
__device__ __forceinline__ v4f mfma(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, AF, BF, 0, 0, 0, 0);
}

// max(a, b, c) of unsigned words as one instruction that the compiler keeps
// where it stands (volatile asm): an unsigned maximum over |x| bit patterns
// is the amax of binary32 values, NaN above +Inf.
__device__ __forceinline__ uint32_t max3_in_place(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm volatile("v_max3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

}  // namespace fp8lin
