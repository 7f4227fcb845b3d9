// gemm_big_kernel.h -- the large-tile FP8 GEMM for gfx950 with block scales
// (k_gemm_big, eight wavefronts), and the tile helpers and epilogue it shares
// with the four-wavefront per-tensor / per-row kernel (gemm_w4_kernel.h):
// kernel and launch templates, instantiated by gemm_big.hip (BF16 / FP32
// output) and gemm_big_fp8out.hip (FP8 output), two translation units
// compiled in parallel.
//
// Same contract as k_gemm in gemm_kernels.hip (see there and the C ABI):
// D = A . B^T, K-contiguous FP8 operands, FP32 accumulation; block scales
// with binary32 values promoted per 128-wide K block (power-of-two ones are
// applied inside the matrix instruction by k_gemm_w4), a per-tensor
// operand's scale folded in.
// [MPG] = "Mixed Precision LLM Training: The Complete Guide",
//   "Skipping the BAcc accumulator promotion", "DeepSeek FP8 training recipe
//   in detail > Block-wise scaling at 128 granularity" and "> Mixed-precision
//   accumulation".
//
// Layout of one workgroup (512 threads, 8 wavefronts):
//   output tile 256 x 256; wavefront w owns rows 128*(w/4).., columns
//   64*(w%4).. (8 x 4 MFMA tiles of 16x16, one v_mfma_f32_16x16x128 per tile
//   per 128-wide K block);
//   K loop in 128-byte steps through two LDS stages of 66 KB (A 32 KB, B
//   32 KB, 1 KB of row scales for each 1x128 operand);
//   operands move global -> LDS with buffer_load_dwordx4 ... lds (no VGPR
//   staging), one instruction per 8 rows x 128 bytes of a tile, so every
//   global read covers whole 128-byte lines.  Tiles are row-major in LDS
//   with 16-byte chunk c of row r stored at chunk c ^ swz(r); a lane's DMA
//   slot is fixed, so the swizzle is applied by choosing which global chunk
//   each lane fetches.  An MFMA operand lane l takes row l % 16 and the K
//   chunks g and g + 4 (g = l / 16); A and B use the same assignment, so
//   every product pairs equal k and each group of 8 consecutive register
//   bytes holds 8 consecutive k.  With this assignment and swz(r) =
//   ((r >> 1) & 7) ^ ((r & 1) << 2) the 16-row ds_read_b128 pattern ran
//   about 1.6x faster than with chunk pairs {2g, 2g+1} (measured on gfx950).
//   Buffer loads past the end of an operand return zeros, which covers the
//   M / N tails without branches (block scales make K a multiple of the
//   step).
//   The prefetch is issued from inline assembly: the compiler then neither
//   waits for it before reading the other stage nor keeps it ordered with
//   anything else; it is spread over the step's first row-tiles, and each
//   step ends with an explicit vmcnt(0) and a barrier.
//   Inside the loop there is no other vector-memory access: per-K-block
//   scales come from LDS (1x128 rows arrive with the operands; per-tensor and
//   128x128 scales sit in a per-wavefront table filled before the loop).
// Workgroup order: the hardware hands consecutive workgroups to the 8 XCDs in
// turn; ids are remapped so each XCD gets a contiguous run of tiles, taken
// 8 tile-rows at a time, so the A and B panels a tile needs sit in that
// XCD's L2.
#pragma once

#include <type_traits>

#include "fp8_device.h"
#include "launch.h"

namespace fp8lin {

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int THREADS = 512, NWAVES = 8;
constexpr int WTM = 128, WTN = 64;       // wavefront tile
constexpr int TI = WTM / 16, TJ = WTN / 16;
constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;
constexpr int SA_OFF = A_BYTES + B_BYTES;
constexpr int SB_OFF = SA_OFF + BM * 4;
constexpr int STAGE = SB_OFF + BN * 4;
constexpr int MAX_KB = 512;              // per-wavefront scale table: K <= 65536
constexpr int GROUP_M = 8;
constexpr uint32_t kOOB = 0x7FFFFFF0u;   // a buffer offset past any operand
constexpr int kRsrcWord3 = 0x00020000;

// The same instruction with per-lane E8M0 block scales: lane l of operand
// `a` holds one row and applies 2^(sa - 127) to it, likewise for `b`.
template <int AF, int BF>
__device__ __forceinline__ v4f mfma_mx(const v8i& a, const v8i& b, const v4f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, AF, BF, 0, sa, 0, sb);
}

// E8M0 code of a power of two 2^e (|e| <= 126): its binary32 exponent field.
__device__ __forceinline__ int e8m0_of(float pow2) { return (int)(__float_as_uint(pow2) >> 23) & 0xFF; }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two binary32 values -> two bf16 (a in the low half) with one
// v_cvt_pk_bf16_f32: round to nearest even, except that the instruction does
// not round binary32 subnormal inputs to nearest (measured over all 2^32
// inputs: every other input, NaN included, matches f32_to_bf16_rne).  The
// caller handles subnormals with f32_to_bf16_rne.
__device__ __forceinline__ uint32_t bf16x2_hw(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Raw buffer resource (wave-uniform): base, no stride, `bytes` records.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(a & 0xFFFFFFFFu));
  r.y = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFFu));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = kRsrcWord3;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint8_t*)p));
}

// 16 bytes per lane from buffer offset `off` into LDS at m0 + 16 * lane.
__device__ __forceinline__ void dma16(uint32_t m0, uint32_t off, i32x4 rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(m0), "v"(off), "s"(rsrc) : "memory", "m0");
}
// The same with the instruction's scalar offset added (the K offset of a
// step, so the lane offsets stay loop-invariant).
__device__ __forceinline__ void dma16s(uint32_t m0, uint32_t off, i32x4 rsrc, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(m0), "v"(off), "s"(rsrc), "s"(soff) : "memory", "m0");
}
// 4 bytes per lane into LDS at m0 + 4 * lane.
__device__ __forceinline__ void dma4(uint32_t m0, uint32_t off, i32x4 rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(m0), "v"(off), "s"(rsrc) : "memory", "m0");
}

__device__ __forceinline__ int swz(int row) { return ((row >> 1) & 7) ^ ((row & 1) << 2); }

// MFMA operand fragment of tile row `row` for lane group g: chunks g, g + 4.
__device__ __forceinline__ v8i frag(const uint8_t* tile, int row, int g) {
  const int sw = swz(row);
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + row * BK + ((g ^ sw) << 4));
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + row * BK + (((g + 4) ^ sw) << 4));
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// ---- epilogue pieces shared by the GEMM kernels.  A wavefront's tile is
// TI x TJ MFMA tiles of 16 x 16 from row r0, column c0 of D; lane (g, l16)
// holds, for each (i, j), D row r0 + 16 i + l16, columns c0 + 16 j + 4 g ..
// +3.  deq(i, j, q, a) dequantises accumulator entry (i, j, q).

// Tile wholly inside D with 16-byte-aligned rows, BF16 or FP32 output:
// staged through the wavefront's REGION bytes of LDS (16-byte chunk c of
// tile row r at chunk c ^ (r & 7)) and written as whole rows, 16 bytes per
// lane (passes of as many rows as the region holds); FP32 `accumulate` adds
// the old row in the same pass.  Returns the running |D| maximum (binary32
// bit pattern; for BF16 the rounded values').
template <int TI, int TJ, int REGION, typename Deq>
__device__ __forceinline__ uint32_t store_staged(const GemmParams& p, const v4f (&acc)[TI][TJ],
                                                 Deq&& deq, bool may_sub, int64_t r0, int64_t c0,
                                                 int lane, uint8_t* wl) {
  constexpr int WTM = 16 * TI, WTN = 16 * TJ;
  const int g = lane >> 4, l16 = lane & 15;
  uint32_t amax_bits = 0;
  auto epi = [&](auto f32tag) {
    constexpr bool F32 = decltype(f32tag)::value;
    constexpr int ES = F32 ? 4 : 2;
    constexpr int ROW_BYTES = WTN * ES;
    constexpr int ROWS_PASS = REGION / ROW_BYTES < WTM ? REGION / ROW_BYTES : WTM;
    constexpr int LANES_ROW = ROW_BYTES / 16;
    constexpr int ROWS_INST = 64 / LANES_ROW;
    static_assert(WTM % ROWS_PASS == 0 && ROWS_PASS % 16 == 0 && ROW_BYTES >= 128, "staging layout");
#pragma unroll
    for (int pass = 0; pass < WTM / ROWS_PASS; ++pass) {
      // BF16: the hardware pair conversion, one row-tile at a time; a
      // row-tile in which any lane holds a binary32 subnormal (which that
      // instruction does not round to nearest) is written again with the
      // integer rounding.  CHK = false: no output can be subnormal, the
      // per-value check is left out.
      auto row_tiles = [&](auto chktag) {
        constexpr bool CHK = decltype(chktag)::value;
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          if ((16 * i) / ROWS_PASS != pass) continue;
          const int r = 16 * i + l16 - pass * ROWS_PASS;
          auto put = [&](auto softtag) -> bool {
            constexpr bool SOFT = decltype(softtag)::value;
            bool sub = false;
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
              float v[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) v[q] = deq(i, j, q, acc[i][j][q]);
              const int byte = (16 * j + 4 * g) * ES;
              uint8_t* dst = wl + r * ROW_BYTES + (((byte >> 4) ^ (r & 7)) << 4) + (byte & 15);
              if constexpr (F32) {
                *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
              } else if constexpr (SOFT) {
                *reinterpret_cast<uint2*>(dst) = make_uint2(
                    (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16),
                    (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16));
              } else {
                if constexpr (CHK) {
#pragma unroll
                  for (int q = 0; q < 4; ++q) sub |= __builtin_isfpclass(v[q], 0x90);
                }
                *reinterpret_cast<uint2*>(dst) =
                    make_uint2(bf16x2_hw(v[0], v[1]), bf16x2_hw(v[2], v[3]));
              }
            }
            return sub;
          };
          const bool sub = put(std::false_type{});
          if constexpr (!F32 && CHK)
            if (__builtin_expect(__any(sub), 0)) put(std::true_type{});
        }
      };
      if (F32 || !may_sub) row_tiles(std::false_type{});
      else row_tiles(std::true_type{});
      // read back whole rows (same wavefront: LDS operations stay in order)
      const int q = lane % LANES_ROW, rr = lane / LANES_ROW;
#pragma unroll 4
      for (int t = 0; t < ROWS_PASS / ROWS_INST; ++t) {
        const int r = t * ROWS_INST + rr;
        uint4 w = *reinterpret_cast<const uint4*>(wl + r * ROW_BYTES + ((q ^ (r & 7)) << 4));
        const int64_t gm = r0 + pass * ROWS_PASS + r;
        uint8_t* gp = reinterpret_cast<uint8_t*>(p.D) + (gm * p.ldd + c0) * ES + q * 16;
        if constexpr (F32) {
          if (p.accumulate) {
            const float4 o = *reinterpret_cast<const float4*>(gp);
            w.x = __float_as_uint(o.x + __uint_as_float(w.x));
            w.y = __float_as_uint(o.y + __uint_as_float(w.y));
            w.z = __float_as_uint(o.z + __uint_as_float(w.z));
            w.w = __float_as_uint(o.w + __uint_as_float(w.w));
          }
          if (p.d_amax) {
            const uint32_t m4[4] = {w.x & 0x7FFFFFFFu, w.y & 0x7FFFFFFFu, w.z & 0x7FFFFFFFu,
                                    w.w & 0x7FFFFFFFu};
#pragma unroll
            for (int e = 0; e < 4; ++e) amax_bits = m4[e] > amax_bits ? m4[e] : amax_bits;
          }
        } else if (p.d_amax) {
          const uint32_t m = absmax_fold(absmax_pk(absmax_pk(absmax_pk(absmax_pk(0u, w.x), w.y), w.z), w.w));
          amax_bits = m > amax_bits ? m : amax_bits;
        }
        *reinterpret_cast<uint4*>(gp) = w;
      }
    }
  };
  if (p.d_f32) epi(std::true_type{});
  else epi(std::false_type{});
  return amax_bits;
}

// Tile wholly inside D (and D_t) with 16-byte-aligned rows, FP8 output:
// codes encode(fl32(v * so)) of the dequantised value v, running maximum of
// |v| (binary32 bit pattern).  The tile goes in PASSES passes of row-tiles;
// each pass's codes are staged row-major (16 TJ bytes per tile row, 16-byte
// chunk c at c ^ (r mod chunks per row)) and leave as whole rows, then go
// into the column-major copy (row stride 144 bytes, 128 rows), which leaves
// as rows of D_t after the last pass.  One pass reuses one area for both
// layouts (max(16 TJ * 128, 16 TJ * 144) bytes of region); more passes keep
// the column-major copy (16 TJ * 144 bytes) beside a row-major area of one
// pass, fewer codes live at a time.
template <int TI, int TJ, int PASSES, typename Deq>
__device__ __forceinline__ uint32_t store_staged8(const GemmParams& p, const v4f (&acc)[TI][TJ],
                                                  Deq&& deq, float so, int64_t r0, int64_t c0,
                                                  int lane, uint8_t* wl) {
  constexpr int WTM = 16 * TI, WTN = 16 * TJ;
  constexpr int CH = WTN / 16;        // 16-byte chunks per row-major row
  constexpr int RPI = 64 / CH;        // rows per read-back instruction
  constexpr int PI = TI / PASSES;     // row-tiles per pass
  constexpr int RM = PASSES == 1 ? 0 : WTN * 144;   // offset of the row-major area
  static_assert(WTM == 128 && TI % PASSES == 0 && (16 * PI) % RPI == 0, "staging layout");
  const int g = lane >> 4, l16 = lane & 15;
  uint32_t amax_bits = 0;
  auto epi8 = [&](auto fmttag) {
    constexpr int F = decltype(fmttag)::value;
    // quad lane t of the transposed copy and its byte selects
    const int t = l16 & 3, k4 = l16 >> 2;
    const uint32_t sel_a = (t & 1) ? (uint32_t)((t + 4) | (t << 8)) : (uint32_t)(t | ((t + 4) << 8));
    const uint32_t sel_f = t < 2 ? 0x05040100u : 0x01000504u;
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      uint32_t code[PI][TJ];
#pragma unroll
      for (int il = 0; il < PI; ++il)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int i = pass * PI + il;
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = deq(i, j, q, acc[i][j][q]);
          // The running maximum is taken here, in place: left to itself the
          // compiler moves it past the NaN-patch branches to the end of the
          // pass, which keeps all the dequantised values live (and spilled).
          amax_bits = max3_in_place(max3_in_place(amax_bits, __float_as_uint(v[0]) & 0x7FFFFFFFu,
                                                  __float_as_uint(v[1]) & 0x7FFFFFFFu),
                                    __float_as_uint(v[2]) & 0x7FFFFFFFu,
                                    __float_as_uint(v[3]) & 0x7FFFFFFFu);
          code[il][j] = cvt4<F, true>(v[0] * so, v[1] * so, v[2] * so, v[3] * so);
          const int r = 16 * il + l16;
          *reinterpret_cast<uint32_t*>(wl + RM + r * WTN + ((j ^ (r & (CH - 1))) << 4) + 4 * g) =
              code[il][j];
        }
      {
        const int q = lane % CH, rr = lane / CH;
#pragma unroll
        for (int u = 0; u < 16 * PI / RPI; ++u) {
          const int r = RPI * u + rr;
          const uint4 w = *reinterpret_cast<const uint4*>(wl + RM + r * WTN + ((q ^ (r & (CH - 1))) << 4));
          uint8_t* gp = reinterpret_cast<uint8_t*>(p.D) + (r0 + 16 * PI * pass + r) * p.ldd + c0 + q * 16;
          *reinterpret_cast<uint4*>(gp) = w;
        }
      }
      if (p.D_t) {
        // Transposed copy: a 4 x 4 byte transpose across each quad of lanes
        // (same g, rows 16i + 4k .. +3): quad lane t gathers byte t of the
        // four lanes' words (DPP quad permutes, then two byte selects), i.e.
        // column 16j + 4g + t, rows 16i + 4k .. +3, and writes them as one
        // dword of the column-major tile (row stride 144 bytes: the 64 lanes
        // hit 64 different banks).  Same wavefront, LDS operations in order:
        // with one pass the row-major reads above complete before these
        // writes reuse the area.
#pragma unroll
        for (int il = 0; il < PI; ++il)
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
            const uint32_t a0 = code[il][j];
            const uint32_t a1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)a0, 0xB1, 0xF, 0xF, false);
            const uint32_t a2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)a0, 0x4E, 0xF, 0xF, false);
            const uint32_t a3 = (uint32_t)__builtin_amdgcn_mov_dpp((int)a0, 0x1B, 0xF, 0xF, false);
            const uint32_t p01 = __builtin_amdgcn_perm(a1, a0, sel_a);
            const uint32_t p23 = __builtin_amdgcn_perm(a3, a2, sel_a);
            *reinterpret_cast<uint32_t*>(wl + (16 * j + 4 * g + t) * 144 + 16 * (pass * PI + il) + 4 * k4) =
                __builtin_amdgcn_perm(p23, p01, sel_f);
          }
      }
    }
    if (p.D_t) {
      const int c = lane & 7, rr = lane >> 3;
#pragma unroll
      for (int u = 0; u < WTN / 8; ++u) {
        const int n = 8 * u + rr;
        const uint4 w = *reinterpret_cast<const uint4*>(wl + n * 144 + 16 * c);
        uint8_t* gp = p.D_t + (c0 + n) * p.ldt + r0 + 16 * c;
        *reinterpret_cast<uint4*>(gp) = w;
      }
    }
  };
  if (p.d_fp8 == 1) epi8(std::integral_constant<int, 0>{});
  else epi8(std::integral_constant<int, 1>{});
  return amax_bits;
}

// f(integral_constant<int, I>) for I = B .. E-1: the index is a constant
// expression whatever the unroller decides, so an array indexed by it stays
// in registers.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Any other tile: element by element with bounds checks (BF16, FP32 or,
// with OUT8, FP8 codes of fl32(v * so) and their transposed copy).
template <int TI, int TJ, bool OUT8, typename Deq>
__device__ __forceinline__ uint32_t store_edge(const GemmParams& p, const v4f (&acc)[TI][TJ],
                                               Deq&& deq, float so, int64_t r0, int64_t c0,
                                               int lane) {
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t M = p.M, N = p.N;
  const int64_t mr0 = r0 + l16, nc0 = c0 + 4 * g;
  uint32_t amax_bits = 0;
  static_for<0, TI>([&](auto itag) {
    constexpr int i = decltype(itag)::value;
    static_for<0, TJ>([&](auto jtag) {
      constexpr int j = decltype(jtag)::value;
      const int64_t m = mr0 + 16 * i, n = nc0 + 16 * j;
      if (m >= M) return;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (n + r >= N) continue;
        float x = deq(i, j, r, acc[i][j][r]);
        if (OUT8) {
          const float xs = x * so;
          const uint8_t c = (uint8_t)((p.d_fp8 == 1 ? cvt4<0, true>(xs, 0.f, 0.f, 0.f)
                                                    : cvt4<1, true>(xs, 0.f, 0.f, 0.f)) & 0xFFu);
          reinterpret_cast<uint8_t*>(p.D)[m * p.ldd + n + r] = c;
          if (p.D_t) p.D_t[(n + r) * p.ldt + m] = c;
          const uint32_t b = __float_as_uint(x) & 0x7FFFFFFFu;
          amax_bits = b > amax_bits ? b : amax_bits;
        } else if (p.d_f32) {
          float* d = reinterpret_cast<float*>(p.D) + m * p.ldd + n + r;
          if (p.accumulate) x = *d + x;
          *d = x;
          const uint32_t b = __float_as_uint(x) & 0x7FFFFFFFu;
          amax_bits = b > amax_bits ? b : amax_bits;
        } else {
          const uint16_t h = f32_to_bf16_rne(x);
          reinterpret_cast<uint16_t*>(p.D)[m * p.ldd + n + r] = h;
          const uint32_t b = (uint32_t)(h & 0x7FFFu) << 16;
          amax_bits = b > amax_bits ? b : amax_bits;
        }
      }
    });
  });
  return amax_bits;
}

// The workgroup's |D| maximum into *d_amax: one device atomic per workgroup.
template <int NW>
__device__ __forceinline__ void workgroup_amax(float* d_amax, uint32_t amax_bits, int lane, int wave) {
  __shared__ uint32_t wmax[NW];
  amax_bits = wave_max_u32(amax_bits);
  if (lane == 0) wmax[wave] = amax_bits;
  __syncthreads();
  if (wave == 0 && lane == 0) {
    uint32_t m = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) m = wmax[w] > m ? wmax[w] : m;
    if (m != 0u) atomic_max_bits(d_amax, m);
  }
}

// The block-scaled GEMM with binary32 block scales, promoted in FP32 per
// 128-wide K block (per-tensor, per-row and power-of-two block scales go to
// k_gemm_w4):
// BLOCK  : always true here (block scales on at least one operand);
// SA_ROWS: A has 1x128 scales (one per row and K block), else one per wave;
// SB_COL : B has 1x128 scales (one per column and K block), else one per wave;
// MX     : always false here.
template <int AF, int BF, bool BLOCK, bool SA_ROWS, bool SB_COL, bool MX, bool OUT8>
__global__ void __launch_bounds__(THREADS) k_gemm_big(GemmParams p, int tiles_m, int tiles_n) {
  static_assert(BLOCK && !MX, "per-tensor, per-row and power-of-two scales run on k_gemm_w4");
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][STAGE];
  __shared__ float su_tab[NWAVES][MAX_KB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
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
  // DMA: wave w fills rows 32w .. 32w+31 of A and of B, 8 rows per
  // instruction; lane p lands in row 8*it + (p >> 3), stored chunk p & 7
  const int lrow = 32 * wave + (lane >> 3);

  // DMA instruction q of a stage (0..3: A rows lrow + 8 q, 4..7: B rows
  // lrow + 8 (q - 4)).  Block scales make K a multiple of the step: every
  // chunk of a step is inside K, and the step's K offset goes in the scalar
  // offset (no per-step VALU work beside the promotion; measured 1-2% on
  // the transformer-block shapes).  Rows past the operand's end fail the
  // buffer range check on the lane offset and read zeros.
  auto load_part = [&](int kb, uint8_t* base, int q) {
    const uint32_t lb = lds_addr(base);
    const int it = q & 3;
    const int row = lrow + 8 * it;
    const int kc = 16 * ((lane & 7) ^ swz(row));
    if (q < 4)
      dma16s(lb + (32 * wave + 8 * it) * BK, (uint32_t)(row * lda + kc), ra, (uint32_t)(kb * BK));
    else
      dma16s(lb + A_BYTES + (32 * wave + 8 * it) * BK, (uint32_t)(row * ldb + kc), rb,
             (uint32_t)(kb * BK));
  };
  auto load_scales = [&](int kb, uint8_t* base) {
    const uint32_t lb = lds_addr(base);
    if constexpr (SA_ROWS) {
      if (wave == 0) {   // 256 row scales of this K block
        const i32x4 rs = make_rsrc(p.a_sinv + (int64_t)kb * M + m0, (uint32_t)(rows_a * 4));
#pragma unroll
        for (int q = 0; q < 4; ++q) dma4(lb + SA_OFF + q * 256, (uint32_t)(q * 256 + lane * 4), rs);
      }
    }
    if constexpr (SB_COL) {
      if (wave == 1) {   // 256 column scales of this K block
        const i32x4 rs = make_rsrc(p.b_sinv + (int64_t)kb * N + n0, (uint32_t)(rows_b * 4));
#pragma unroll
        for (int q = 0; q < 4; ++q) dma4(lb + SB_OFF + q * 256, (uint32_t)(q * 256 + lane * 4), rs);
      }
    }
  };
  auto load_stage = [&](int kb, uint8_t* base) {
#pragma unroll
    for (int q = 0; q < 8; ++q) load_part(kb, base, q);
    load_scales(kb, base);
  };

  v4f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // The FP8 output scale is read now, ahead of the first DMA: the wait for
  // stage 0 covers it, and the epilogue does not start with a round trip
  // to memory.
  float so = 1.0f;
  if constexpr (OUT8) so = p.d_scale[0];

  // the first two stages go out together, so the second one's latency
  // overlaps the first's; the loop's first step then issues no DMA
  load_stage(0, lds[0]);
  if (nk > 1) load_stage(1, lds[1]);

  // ---- per-wavefront table of the uniform part of each K block's scale
  if constexpr (!(SA_ROWS && SB_COL)) {
    const int64_t mb = min((m0 + wm * WTM) / 128, (M + 127) / 128 - 1);
    const int64_t nb = min((n0 + wn * WTN) / 128, (N + 127) / 128 - 1);
    for (int kb = lane; kb < nk; kb += 64) {
      float s = 1.0f;
      if constexpr (!SA_ROWS)
        s = p.a_scaling == 0 ? p.a_sinv[0] : p.a_sinv[kb * ((M + 127) / 128) + mb];
      if constexpr (!SB_COL)
        s *= p.b_scaling == 0 ? p.b_sinv[0] : p.b_sinv[kb * ((N + 127) / 128) + nb];
      su_tab[wave][kb] = s;
    }
  }

  // stage 0 only: at most 8 DMAs of stage 1 may remain (the wavefronts that
  // also load scales have 12 in stage 1 and wait for 4 of them as well;
  // loads count down in issue order)
  if (nk > 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int kb = 0; kb < nk; ++kb) {
    const int stage = kb & 1;
    const uint8_t* As = lds[stage];
    const uint8_t* Bs = As + A_BYTES;

    // fragment reads first (A row-tile 0 with B column-tile 0 ahead of the
    // rest, so the first MFMA can start early), then the next stage's DMA:
    // after the barrier every wavefront wants its fragments at once, and
    // DMA instructions issued ahead of them delay them (measured: 2-4%
    // faster than issuing the DMA first)
    const v8i a_first = frag(As, wm * WTM + l16, g);
    v8i bfr[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j) bfr[j] = frag(Bs, wn * WTN + 16 * j + l16, g);
    // the next stage's DMA goes into the stage the previous step read (the
    // end-of-step barrier freed it): the scales now, the operands spread
    // over the first row-tiles below.  Issued right after that barrier,
    // its longer-lived addresses push the promotion kernels past 256
    // registers (measured: spills).
    const bool dma = kb > 0 && kb + 1 < nk;
    if (dma) load_scales(kb + 1, lds[stage ^ 1]);

    // The MFMA takes B as its first operand, so each 16x16 result tile is
    // the transpose of the D tile: lane (g, l16) holds D row 16*i + l16,
    // columns 16*j + 4*g .. +3 -- four consecutive outputs of one row.
    {
      float scol[TJ][4];
      if constexpr (SB_COL) {
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const float4 sv =
              *reinterpret_cast<const float4*>(As + SB_OFF + (wn * WTN + 16 * j + 4 * g) * 4);
          scol[j][0] = sv.x; scol[j][1] = sv.y; scol[j][2] = sv.z; scol[j][3] = sv.w;
        }
      }
      float suni = 1.0f;
      if constexpr (!(SA_ROWS && SB_COL)) suni = su_tab[wave][kb];
      // one row-tile at a time: the next A fragment is read while this
      // tile's MFMAs run, and the block partials of the previous row-tile
      // are promoted while this row's MFMAs execute (their results are
      // long ready by then); the last row is promoted after the loop.  The
      // scheduling barrier keeps each row's MFMAs ahead of the promotion.
      auto promote = [&](int i, const v4f (&pp)[TJ], float sr) {
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if constexpr (SB_COL)
              acc[i][j][r] = __builtin_fmaf(pp[j][r] * sr, scol[j][r], acc[i][j][r]);
            else
              acc[i][j][r] = __builtin_fmaf(pp[j][r], sr, acc[i][j][r]);
          }
      };
      v8i a_cur = a_first;
      v4f pprev[TJ];
      float sprev = 0.0f;
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        v8i a_nxt = a_cur;
        if (i + 1 < TI) a_nxt = frag(As, wm * WTM + 16 * (i + 1) + l16, g);
        float srow = suni;
        if constexpr (SA_ROWS) {
          srow = reinterpret_cast<const float*>(As + SA_OFF)[wm * WTM + 16 * i + l16];
          if constexpr (!SB_COL) srow *= suni;
        }
        // the next stage's operand DMA, PER instructions with each of the
        // first 8 / PER row-tiles (3-4% faster than all eight at the step's
        // start for FWD / DGRAD, 2% for WGRAD; two per row-tile push the
        // column-scaled kernels past 256 registers)
        constexpr int PER = SB_COL ? 4 : 2;
        if (dma && i < 8 / PER) {
#pragma unroll
          for (int u = 0; u < PER; ++u) load_part(kb + 1, lds[stage ^ 1], PER * i + u);
        }
        v4f pcur[TJ];
#pragma unroll
        for (int j = 0; j < TJ; ++j) pcur[j] = mfma<BF, AF>(bfr[j], a_cur, v4f{0.f, 0.f, 0.f, 0.f});
        if (i > 0) promote(i - 1, pprev, sprev);
#pragma unroll
        for (int j = 0; j < TJ; ++j) pprev[j] = pcur[j];
        sprev = srow;
        a_cur = a_nxt;
        // one matrix instruction, then its share of the promotion
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, SB_COL ? 8 : 4, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      promote(TI - 1, pprev, sprev);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // ---- epilogue.  Lane (g, l16) holds, for each (i, j), D row 16*i + l16,
  // columns 16*j + 4*g .. +3 of the wavefront's 128 x 64 tile.  Tiles wholly
  // inside D with 16-byte-aligned rows are staged through LDS (each
  // wavefront owns 16 KB of the freed operand stages: 16-byte chunk c of
  // tile row r sits at chunk c ^ (r & 7)) and leave as whole rows, 16 bytes
  // per lane: one 128-byte line per tile row for BF16, two for FP32 (FP32
  // goes in two passes of 64 rows).  Other tiles store element by element
  // with bounds checks.  Block scales can make any output a binary32
  // subnormal, so the BF16 conversion always checks for them.
  const bool may_sub = true;
  // dequantised value of accumulator entry (i, j, q): the promoted
  // accumulators carry their scales
  auto deq = [&](int, int, int, float a) -> float { return a; };
  const int esz = OUT8 ? 1 : (p.d_f32 ? 4 : 2);
  const bool staged = (m0 + BM <= M) && (n0 + BN <= N) && ((p.ldd * esz) % 16 == 0) &&
                      ((reinterpret_cast<uintptr_t>(p.D) & 15u) == 0) &&
                      (p.D_t == nullptr || ((p.ldt % 16 == 0) &&
                                            ((reinterpret_cast<uintptr_t>(p.D_t) & 15u) == 0)));
  uint32_t amax_bits = 0;
  if (OUT8 && staged) {
    __syncthreads();   // every wavefront is done reading both stages
    amax_bits = store_staged8<TI, TJ, 1>(p, acc, deq, so, m0 + wm * WTM, n0 + wn * WTN, lane,
                                      &lds[0][0] + wave * 16384);
  } else if (staged) {
    __syncthreads();   // every wavefront is done reading both stages
    amax_bits = store_staged<TI, TJ, 16384>(p, acc, deq, may_sub, m0 + wm * WTM, n0 + wn * WTN, lane,
                                            &lds[0][0] + wave * 16384);
  } else {
    amax_bits = store_edge<TI, TJ, OUT8>(p, acc, deq, so, m0 + wm * WTM, n0 + wn * WTN, lane);
  }
  if (p.d_amax) workgroup_amax<NWAVES>(p.d_amax, amax_bits, lane, wave);
}

template <int AF, int BF, bool BLOCK, bool SA_ROWS, bool SB_COL, bool MX, bool OUT8>
hipError_t launch_one(const GemmParams& p, hipStream_t s) {
  auto kern = k_gemm_big<AF, BF, BLOCK, SA_ROWS, SB_COL, MX, OUT8>;
  const int tiles_m = (int)((p.M + BM - 1) / BM), tiles_n = (int)((p.N + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3((unsigned)(tiles_m * tiles_n)), dim3(THREADS), 0, s, p, tiles_m,
                     tiles_n);
  return hipGetLastError();
}

template <int AF, int BF, bool MX, bool OUT8>
hipError_t launch_block(const GemmParams& p, hipStream_t s) {
  const bool sa = p.a_scaling == 1 || p.a_scaling == 3, sb = p.b_scaling == 1 || p.b_scaling == 3;
  if (sa && sb) return launch_one<AF, BF, true, true, true, MX, OUT8>(p, s);
  if (sa) return launch_one<AF, BF, true, true, false, MX, OUT8>(p, s);
  if (sb) return launch_one<AF, BF, true, false, true, MX, OUT8>(p, s);
  return launch_one<AF, BF, true, false, false, MX, OUT8>(p, s);
}

// Scaling codes: 0 per-tensor, 1 / 2 block (1x128 / 128x128) with any
// binary32 scales, 3 / 4 the same blocks with power-of-two scales, 5 one
// scale per row (with per-tensor or per-row operands only).  When
// every block-scaled operand has power-of-two scales the block scales go
// into the matrix instruction; otherwise they are promoted in FP32 (a
// power of two is a binary32 scale like any other).
template <int AF, int BF, bool OUT8>
hipError_t launch_fmt(const GemmParams& p, hipStream_t s) {
  // per-tensor, per-row and power-of-two block scales go to the
  // four-wavefront kernel before this point: here at least one operand has
  // block scales with binary32 values, promoted in FP32
  return launch_block<AF, BF, false, OUT8>(p, s);
}

// OUT8: FP8 output (its own instantiations, so that the BF16 / FP32 kernels
// carry none of its registers).
template <bool OUT8>
hipError_t launch_gemm_big_out(const GemmParams& p, hipStream_t s) {
  if (p.a_fmt == 0 && p.b_fmt == 0) return launch_fmt<0, 0, OUT8>(p, s);
  if (p.a_fmt == 1 && p.b_fmt == 0) return launch_fmt<1, 0, OUT8>(p, s);
  if (p.a_fmt == 0 && p.b_fmt == 1) return launch_fmt<0, 1, OUT8>(p, s);
  return launch_fmt<1, 1, OUT8>(p, s);
}

}  // namespace

}  // namespace fp8lin
