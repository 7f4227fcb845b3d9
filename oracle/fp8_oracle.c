/*
 * fp8_oracle.c -- plain, slow CPU oracle for the FP8 scaled linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant
 * generator with the HIP library: every conversion here is written out with
 * integer bit manipulation on IEEE-754 binary32 patterns, and every
 * reduction is a plain loop in the order the method states.
 *
 * Sources (web pages; cited by title and section):
 *   [MPG]  "Mixed Precision LLM Training: The Complete Guide"
 *          (blog.prompt20.com/posts/mixed-precision-training)
 *   [TALK] PyData Amsterdam 2026 talk abstract "FP8 for pretraining"
 *          (pretalx.com), outline 05:00-15:00
 *   [P3]   "Training and inference of large language models using 8-bit
 *          floating point" (arXiv 2309.17224 library entry), abstract
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -pthread -shared -fPIC
 * (contraction off: every float operation below must round on its own).
 */
#include <float.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define O_E4M3 0
#define O_E5M2 1

#define O_SCALE_TENSOR 0
#define O_SCALE_1x128 1
#define O_SCALE_128x128 2
#define O_SCALE_ROW 5   /* one scale per row of an operand, applied after the K sum */

#define O_ALGO_MAX 0
#define O_ALGO_MOST_RECENT 1

/* ------------------------------------------------------------------ */
/* binary32 <-> bits                                                   */
/* ------------------------------------------------------------------ */
static float f_of(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t b_of(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

/* bf16 is the top half of a binary32 pattern: widening is exact. */
float o_bf16_to_f32(uint16_t h) { return f_of((uint32_t)h << 16); }

/* ------------------------------------------------------------------ */
/* FP8 format parameters.                                              */
/* [MPG] "The precision formats" table and the "FP8 E4M3" / "FP8 E5M2"  */
/* entries: E4M3 = 1 sign, 4 exponent, 3 mantissa bits, range about   */
/* 2^-9 .. 448; E5M2 = 1 sign, 5 exponent, 2 mantissa bits, range      */
/* about 2^-16 .. 57344.  Those two maxima and minima fit only the OCP */
/* encodings: E4M3 without infinities (all-ones exponent+mantissa is   */
/* NaN, so the top finite code is 0x7E = 448) and E5M2 with IEEE-style */
/* Inf/NaN (top finite code 0x7B = 57344).                             */
/* ------------------------------------------------------------------ */
typedef struct {
  int ebits, mbits, bias;
  int max_code;   /* largest finite magnitude code */
} fp8_fmt;

static fp8_fmt fmt_of(int fmt) {
  fp8_fmt f;
  if (fmt == O_E4M3) { f.ebits = 4; f.mbits = 3; f.bias = 7;  f.max_code = 0x7E; }
  else               { f.ebits = 5; f.mbits = 2; f.bias = 15; f.max_code = 0x7B; }
  return f;
}

/* Largest finite value of the format (448 or 57344). */
double o_fp8_max(int fmt) { return fmt == O_E4M3 ? 448.0 : 57344.0; }

/* Decode one FP8 code to its exact value (every FP8 value is exact in
 * binary64).  Field split s|e|m; e == 0 is subnormal m*2^(1-bias-M),
 * otherwise (1+m/2^M)*2^(e-bias).  E4M3: e=15,m=7 is NaN, no Inf.
 * E5M2: e=31,m=0 is Inf, e=31,m!=0 is NaN. */
double o_fp8_decode(uint8_t c, int fmt) {
  fp8_fmt f = fmt_of(fmt);
  int s = c >> 7;
  int e = (c >> f.mbits) & ((1 << f.ebits) - 1);
  int m = c & ((1 << f.mbits) - 1);
  double v;
  if (fmt == O_E4M3 && e == 15 && m == 7) return NAN;
  if (fmt == O_E5M2 && e == 31) {
    if (m != 0) return NAN;
    return s ? -INFINITY : INFINITY;
  }
  if (e == 0)
    v = ldexp((double)m, 1 - f.bias - f.mbits);
  else
    v = ldexp(1.0 + (double)m / (double)(1 << f.mbits), e - f.bias);
  return s ? -v : v;
}

/* ------------------------------------------------------------------ */
/* Saturating round-to-nearest-even encoder, by bit manipulation.      */
/*                                                                     */
/* Readings (the pages leave these open):                              */
/*  - rounding: round to nearest, ties to even ([MPG] "Stochastic      */
/*    rounding" contrasts SR with round-to-nearest);                   */
/*  - overflow: [MPG] "Numerical stability deep dive > Overflow" says  */
/*    values past the maximum become infinite; the scaled linear layer  */
/*    here saturates instead: a finite result beyond the largest code   */
/*    and +-Inf both map to +-max;                                     */
/*  - NaN maps to 0x7F | sign (a NaN code in both formats);            */
/*  - the sign is kept on results that round to zero;                  */
/*  - underflow: [MPG] "Underflow" says values below about 2^-9 become */
/*    zero for E4M3; under round-to-nearest-even exactly half the      */
/*    smallest subnormal (2^-10) ties to the even code 0, and anything */
/*    above it rounds up to 2^-9.                                      */
/* ------------------------------------------------------------------ */
uint8_t o_fp8_encode(float x, int fmt) {
  fp8_fmt f = fmt_of(fmt);
  uint32_t u = b_of(x);
  uint32_t sign = (u >> 31) << 7;
  uint32_t a = u & 0x7FFFFFFFu;
  int emin = 1 - f.bias;               /* exponent of the smallest normal */
  uint64_t sig;
  int e, te, shift;
  uint64_t q, rem, half;
  int code;

  if (a > 0x7F800000u) return (uint8_t)(sign | 0x7F);          /* NaN  */
  if (a == 0x7F800000u) return (uint8_t)(sign | f.max_code);   /* +-Inf */

  /* x = sig * 2^(e - 23) exactly. */
  if ((a >> 23) == 0) { sig = a & 0x7FFFFFu; e = -126; }
  else { sig = (a & 0x7FFFFFu) | 0x800000u; e = (int)(a >> 23) - 127; }

  /* Target exponent: the FP8 grid spacing at this magnitude is
   * 2^(te - M) with te = max(e, emin). */
  te = e > emin ? e : emin;
  /* q = x / 2^(te-M) = sig * 2^(e - 23 - te + M) = sig >> shift */
  shift = 23 + te - e - f.mbits;       /* >= 23 - M > 0 */
  if (shift >= 63) {
    q = 0; rem = sig; half = (uint64_t)1 << 62;   /* rem < half: no round */
  } else {
    q = sig >> shift;
    rem = sig & (((uint64_t)1 << shift) - 1);
    half = (uint64_t)1 << (shift - 1);
  }
  if (rem > half || (rem == half && (q & 1))) q += 1;

  /* Code magnitude: ((te - emin) << M) + q covers subnormals (te = emin,
   * q < 2^M), normals (q in [2^M, 2^(M+1))) and the rounding carry
   * (q = 2^(M+1) lands on the next binade) with one formula. */
  code = ((te - emin) << f.mbits) + (int)q;
  if (code > f.max_code) code = f.max_code;                     /* saturate */
  return (uint8_t)(sign | (uint32_t)code);
}

/* ------------------------------------------------------------------ */
/* Amax: max_i |x_i| over a bf16 tensor ([MPG] "Per-tensor scaling":   */
/* the scale is chosen from the tensor's maximum absolute value).      */
/* Reading: the maximum is taken in IEEE totalOrder on magnitudes, so  */
/* a NaN input propagates (NaN sits above +Inf).  For non-negative     */
/* binary32 values totalOrder is the unsigned order of their bit       */
/* patterns, and |x| of a bf16 clears bit 15.                          */
/* ------------------------------------------------------------------ */
float o_amax_bf16(const uint16_t* x, int64_t n) {
  uint32_t best = 0;
  for (int64_t i = 0; i < n; ++i) {
    uint32_t mag = (uint32_t)(x[i] & 0x7FFFu) << 16;   /* bits of |x_i| */
    if (mag > best) best = mag;
  }
  return f_of(best);
}

/* ------------------------------------------------------------------ */
/* Scale from an amax.                                                 */
/* [MPG] "Per-tensor scaling": multiply the tensor by a scale before   */
/* quantising so its amax lands at the top of the FP8 range, and       */
/* multiply the matmul result by the inverse scale.  The recipe exposes */
/* a `margin` (DelayedScaling(margin=0, ...)) without its formula.     */
/* Readings: s = fl32(fmax / amax), then s = s * 2^-margin;            */
/* s_inv = fl32(1 / s).  amax == 0 or non-finite: no valid scale       */
/* ([MPG] "torch.compile and FP8": the scale update is skipped for an  */
/* all-zero tensor) -- the caller keeps `fallback` (1.0 for current    */
/* and block scaling, the previous scale for delayed scaling).  A      */
/* quotient that overflows binary32 is clamped to FLT_MAX.             */
/* Returns 1 if a new scale was computed, 0 if the fallback was kept.  */
/* ------------------------------------------------------------------ */
int o_compute_scale(float amax, int fmt, int margin, float fallback,
                    float* scale, float* scale_inv) {
  float fmax = (float)o_fp8_max(fmt);
  float s;
  if (!(amax > 0.0f) || isinf(amax) || isnan(amax)) {
    *scale = fallback;
    *scale_inv = 1.0f / fallback;
    return 0;
  }
  s = fmax / amax;                       /* IEEE single division, RNE */
  if (isinf(s)) s = FLT_MAX;
  if (margin != 0) s = ldexpf(s, -margin);
  *scale = s;
  *scale_inv = 1.0f / s;
  return 1;
}

/* ------------------------------------------------------------------ */
/* Power-of-two ("exponent bias") scale.                               */
/* [P3] abstract and reviews: the scale is an exponent bias chosen     */
/* from the tensor's maximum (FP8-AMAX) so that its range roughly      */
/* matches the format's.  The page does not print the formula          */
/* (its section 2.3 is not on the page).  Reading: s = 2^e with e the  */
/* largest integer such that amax * 2^e <= fmax (no saturation, the    */
/* amax lands in (fmax/2, fmax]), then e -= margin, e clamped to       */
/* [-126, 126] so s and 1/s are normal binary32 powers of two;         */
/* scale_inv = 2^-e.  Both are exact.  Same fallback rule as           */
/* o_compute_scale for amax == 0 or non-finite.                        */
/* e is found by comparing mantissas after frexp (exact on doubles).   */
/* ------------------------------------------------------------------ */
int o_pow2_exponent(float amax, int fmt) {
  int ea, ef;
  double ma = frexp((double)amax, &ea);          /* amax = ma * 2^ea, ma in [0.5, 1) */
  double mf = frexp(o_fp8_max(fmt), &ef);        /* fmax = mf * 2^ef */
  return ma <= mf ? ef - ea : ef - ea - 1;
}

int o_compute_scale_pow2(float amax, int fmt, int margin, float fallback,
                         float* scale, float* scale_inv) {
  int e;
  if (!(amax > 0.0f) || isinf(amax) || isnan(amax)) {
    *scale = fallback;
    *scale_inv = 1.0f / fallback;
    return 0;
  }
  e = o_pow2_exponent(amax, fmt) - margin;
  if (e > 126) e = 126;
  if (e < -126) e = -126;
  *scale = ldexpf(1.0f, e);
  *scale_inv = ldexpf(1.0f, -e);
  return 1;
}

typedef int (*scale_rule_fn)(float, int, int, float, float*, float*);

/* ------------------------------------------------------------------ */
/* Delayed scaling with an amax history.                               */
/* [MPG] "Delayed scaling (the default recipe)": the scale used at     */
/* step t comes from earlier steps; "History-based scaling": the scale */
/* is set from the max over the last N amaxes (N = 16 by default,      */
/* "amax_compute_algo" = "max", or "most_recent").                     */
/* Readings: history[len] per tensor, newest at index 0; each update   */
/* shifts the history down by one and inserts the new amax; the        */
/* effective amax is the maximum of the whole window (NaN propagates,  */
/* as in o_amax_bf16) or the newest entry; the next scale is           */
/* o_compute_scale(effective amax) with the previous scale as the      */
/* fallback.                                                           */
/* ------------------------------------------------------------------ */
static int tot_gt(float a, float b) {  /* a > b in totalOrder on magnitudes >= 0 */
  return b_of(a) > b_of(b);
}

static void history_update_rule(float* history, int64_t n, int64_t len,
                                const float* amax_new, int fmt, int margin, int algo,
                                float* scale, float* scale_inv, scale_rule_fn rule) {
  for (int64_t t = 0; t < n; ++t) {
    float* h = history + t * len;
    float eff;
    for (int64_t j = len - 1; j >= 1; --j) h[j] = h[j - 1];
    h[0] = amax_new[t];
    if (algo == O_ALGO_MOST_RECENT) {
      eff = h[0];
    } else {
      eff = h[0];
      for (int64_t j = 1; j < len; ++j)
        if (tot_gt(h[j], eff)) eff = h[j];
    }
    rule(eff, fmt, margin, scale[t], &scale[t], &scale_inv[t]);
  }
}

void o_history_update(float* history, int64_t n, int64_t len, const float* amax_new, int fmt,
                      int margin, int algo, float* scale, float* scale_inv) {
  history_update_rule(history, n, len, amax_new, fmt, margin, algo, scale, scale_inv,
                      o_compute_scale);
}

/* The same update with the power-of-two rule (o_compute_scale_pow2). */
void o_history_update_pow2(float* history, int64_t n, int64_t len, const float* amax_new,
                           int fmt, int margin, int algo, float* scale, float* scale_inv) {
  history_update_rule(history, n, len, amax_new, fmt, margin, algo, scale, scale_inv,
                      o_compute_scale_pow2);
}

/* ------------------------------------------------------------------ */
/* Per-tensor scaled cast: q = encode(fl32(x * s)).                    */
/* [MPG] "Per-tensor scaling": multiply by the scale, then quantise.   */
/* Reading: two roundings, a binary32 multiply (RNE) then the          */
/* saturating RNE encode -- not one fused rounding of the exact        */
/* product.  Also records max|x| of the input when amax_out != NULL.   */
/* ------------------------------------------------------------------ */
void o_cast(const uint16_t* x, int64_t n, float s, int fmt, uint8_t* y) {
  for (int64_t i = 0; i < n; ++i) {
    float v = o_bf16_to_f32(x[i]);
    float p = v * s;
    y[i] = o_fp8_encode(p, fmt);
  }
}

/* Saturation and underflow counts of the per-tensor cast, the overflow /
 * underflow ratios of the diagnostic dashboard ([MPG] "Numerical-failure
 * taxonomy > A diagnostic dashboard", quantities per layer).  Reading:
 * with v = fl32(x * s) as in o_cast, an element saturates when |v| is
 * beyond the format's largest finite value (Inf included, NaN not); it
 * underflows when x is nonzero and its code is +-0 -- decided by the
 * encoder itself, not by a threshold.  counts[0] += saturated,
 * counts[1] += underflowed. */
void o_cast_stats(const uint16_t* x, int64_t n, float s, int fmt, uint64_t counts[2]) {
  const double mx = o_fp8_max(fmt);
  for (int64_t i = 0; i < n; ++i) {
    const float p = o_bf16_to_f32(x[i]) * s;
    if (!isnan(p) && fabs((double)p) > mx) counts[0] += 1;
    if ((x[i] & 0x7FFFu) != 0 && (o_fp8_encode(p, fmt) & 0x7Fu) == 0) counts[1] += 1;
  }
}

/* Cast plus transpose: y_t[c][r] = y[r][c] for x laid out [rows][cols].
 * Per-tensor scaling makes the transposed bytes the same bytes. */
void o_cast_transpose(const uint16_t* x, int64_t rows, int64_t cols, float s,
                      int fmt, uint8_t* y, uint8_t* y_t) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      uint8_t q = o_fp8_encode(o_bf16_to_f32(x[r * cols + c]) * s, fmt);
      if (y) y[r * cols + c] = q;
      if (y_t) y_t[c * rows + r] = q;
    }
}

/* ------------------------------------------------------------------ */
/* Block-wise cast.                                                    */
/* [MPG] "DeepSeek FP8 training recipe in detail > Block-wise scaling  */
/* at 128 granularity": one scale per 128x128 block of a weight        */
/* matrix, one per 128-element segment of an activation; the scales    */
/* are computed on the fly and stored next to the data.                */
/* Per tile: amax over the elements present (o_amax), s from           */
/* o_compute_scale with fallback 1.0, then o_cast element-wise.        */
/*                                                                     */
/* x is [rows][cols] row-major bf16.                                   */
/* tile == O_SCALE_1x128:                                              */
/*   y   [rows][cols], one scale per (row, 128 cols):                  */
/*       sinv[cb * rows + r], cb = c / 128   (layout [ceil(cols/128)][rows]) */
/*   y_t [cols][rows], one scale per (col, 128 rows), computed from    */
/*       bf16 (not from y): sinv_t[rb * cols + c]                      */
/*       (layout [ceil(rows/128)][cols]).                              */
/* tile == O_SCALE_128x128:                                            */
/*   one scale per (128-row, 128-col) block; y_t is the byte transpose */
/*   of y; sinv[cb * nrb + rb] (layout [ceil(cols/128)][ceil(rows/128)]) */
/*   and sinv_t[rb * ncb + cb] (layout [ceil(rows/128)][ceil(cols/128)]). */
/* Any of y/sinv/y_t/sinv_t may be NULL.                               */
/* ------------------------------------------------------------------ */
static void cast_block_rule(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int tile,
                            uint8_t* y, float* sinv, uint8_t* y_t, float* sinv_t,
                            scale_rule_fn rule) {
  int64_t nrb = (rows + 127) / 128, ncb = (cols + 127) / 128;
  float s, si;
  if (tile == O_SCALE_1x128) {
    /* row-wise segments along cols */
    for (int64_t r = 0; r < rows; ++r)
      for (int64_t cb = 0; cb < ncb; ++cb) {
        int64_t c0 = cb * 128, c1 = c0 + 128 < cols ? c0 + 128 : cols;
        float am = o_amax_bf16(x + r * cols + c0, c1 - c0);
        rule(am, fmt, 0, 1.0f, &s, &si);
        if (sinv) sinv[cb * rows + r] = si;
        if (y)
          for (int64_t c = c0; c < c1; ++c)
            y[r * cols + c] = o_fp8_encode(o_bf16_to_f32(x[r * cols + c]) * s, fmt);
      }
    /* column-wise segments along rows, for the transposed copy */
    if (y_t || sinv_t) {
      uint16_t seg[128];
      for (int64_t c = 0; c < cols; ++c)
        for (int64_t rb = 0; rb < nrb; ++rb) {
          int64_t r0 = rb * 128, r1 = r0 + 128 < rows ? r0 + 128 : rows;
          for (int64_t r = r0; r < r1; ++r) seg[r - r0] = x[r * cols + c];
          float am = o_amax_bf16(seg, r1 - r0);
          rule(am, fmt, 0, 1.0f, &s, &si);
          if (sinv_t) sinv_t[rb * cols + c] = si;
          if (y_t)
            for (int64_t r = r0; r < r1; ++r)
              y_t[c * rows + r] = o_fp8_encode(o_bf16_to_f32(x[r * cols + c]) * s, fmt);
        }
    }
  } else {
    for (int64_t rb = 0; rb < nrb; ++rb)
      for (int64_t cb = 0; cb < ncb; ++cb) {
        int64_t r0 = rb * 128, r1 = r0 + 128 < rows ? r0 + 128 : rows;
        int64_t c0 = cb * 128, c1 = c0 + 128 < cols ? c0 + 128 : cols;
        float am = 0.0f;
        for (int64_t r = r0; r < r1; ++r) {
          float m = o_amax_bf16(x + r * cols + c0, c1 - c0);
          if (tot_gt(m, am)) am = m;
        }
        rule(am, fmt, 0, 1.0f, &s, &si);
        if (sinv) sinv[cb * nrb + rb] = si;
        if (sinv_t) sinv_t[rb * ncb + cb] = si;
        for (int64_t r = r0; r < r1; ++r)
          for (int64_t c = c0; c < c1; ++c) {
            uint8_t q = o_fp8_encode(o_bf16_to_f32(x[r * cols + c]) * s, fmt);
            if (y) y[r * cols + c] = q;
            if (y_t) y_t[c * rows + r] = q;
          }
      }
  }
}

void o_cast_block(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int tile,
                  uint8_t* y, float* sinv, uint8_t* y_t, float* sinv_t) {
  cast_block_rule(x, rows, cols, fmt, tile, y, sinv, y_t, sinv_t, o_compute_scale);
}

/* The same tiles with power-of-two scales (o_compute_scale_pow2). */
void o_cast_block_pow2(const uint16_t* x, int64_t rows, int64_t cols, int fmt, int tile,
                       uint8_t* y, float* sinv, uint8_t* y_t, float* sinv_t) {
  cast_block_rule(x, rows, cols, fmt, tile, y, sinv, y_t, sinv_t, o_compute_scale_pow2);
}

/* ------------------------------------------------------------------ */
/* Row-wise cast.                                                      */
/* [MPG] "Per-row vs per-tensor scaling": one scale per row (per       */
/* output channel of a weight, per token of an activation), a middle   */
/* ground between one scale per tensor and block scales.               */
/* y [rows][cols]: each row r with s = o_compute_scale(amax of row r,  */
/* fallback 1); sinv[r] = 1/s.                                         */
/* y_t [cols][rows]: each column c of x (a row of the transposed       */
/* operand) with its own scale from the column's amax; sinv_t[c].      */
/* Either pair may be NULL.                                            */
/* ------------------------------------------------------------------ */
void o_cast_rowwise(const uint16_t* x, int64_t rows, int64_t cols, int fmt, uint8_t* y,
                    float* sinv, uint8_t* y_t, float* sinv_t) {
  float s, si;
  if (y || sinv)
    for (int64_t r = 0; r < rows; ++r) {
      float am = o_amax_bf16(x + r * cols, cols);
      o_compute_scale(am, fmt, 0, 1.0f, &s, &si);
      if (sinv) sinv[r] = si;
      if (y)
        for (int64_t c = 0; c < cols; ++c)
          y[r * cols + c] = o_fp8_encode(o_bf16_to_f32(x[r * cols + c]) * s, fmt);
    }
  if (y_t || sinv_t)
    for (int64_t c = 0; c < cols; ++c) {
      float am = 0.0f;
      for (int64_t r = 0; r < rows; ++r) {
        float m = o_amax_bf16(x + r * cols + c, 1);
        if (tot_gt(m, am)) am = m;
      }
      o_compute_scale(am, fmt, 0, 1.0f, &s, &si);
      if (sinv_t) sinv_t[c] = si;
      if (y_t)
        for (int64_t r = 0; r < rows; ++r)
          y_t[c * rows + r] = o_fp8_encode(o_bf16_to_f32(x[r * cols + c]) * s, fmt);
    }
}

/* ------------------------------------------------------------------ */
/* Stochastic rounding.                                                */
/* [MPG] "Stochastic rounding": instead of rounding to nearest, round  */
/* up or down at random according to the remainder, which makes the   */
/* rounded value unbiased.  [TALK] outline: "rounding techniques".     */
/*                                                                     */
/* Random words: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel  */
/* random numbers: as easy as 1, 2, 3", SC 2011), a counter-based      */
/* generator: ten rounds of two 32x32->64 multiplications whose halves */
/* are mixed with the other words and the round key; the key advances  */
/* by the two Weyl constants after each round.                          */
/* ------------------------------------------------------------------ */
void o_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    uint64_t p0 = (uint64_t)0xD2511F53u * c0;   /* the two multipliers of Philox4x32 */
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    uint32_t n1 = (uint32_t)p1;
    uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    uint32_t n3 = (uint32_t)p0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += 0x9E3779B9u;                          /* golden ratio */
    k1 += 0xBB67AE85u;                          /* sqrt(3) - 1 */
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The random word of element i of a tensor (row-major index) under
 * (seed, offset): word i % 4 of Philox4x32-10 with counter
 * (i / 4, offset) as four little-endian 32-bit words and key seed. */
uint32_t o_sr_word(uint64_t seed, uint64_t offset, uint64_t i) {
  uint64_t g = i >> 2;
  uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), (uint32_t)offset, (uint32_t)(offset >> 32)};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  o_philox4x32_10(ctr, key, out);
  return out[i & 3];
}

/* Stochastic rounding of a binary32 value to an FP8 code with the random
 * word r.  |v| >= fmax and +-Inf saturate to +-fmax, NaN gives 0x7F|sign
 * (as the round-to-nearest encoder).  Otherwise, with lo the largest FP8
 * magnitude <= |v| and hi the next one, the magnitude becomes hi when
 * r < (|v| - lo) / (hi - lo) * 2^32 (probability (|v| - lo) / (hi - lo)
 * for a uniform r, exactly when that ratio is a multiple of 2^-32), else
 * lo; the sign of v is kept.  lo is found by a search over the codes. */
uint8_t o_fp8_encode_sr(float v, int fmt, uint32_t r) {
  uint32_t sign = (b_of(v) >> 31) ? 0x80u : 0x00u;
  double a = fabs((double)v);
  double fmax = o_fp8_max(fmt);
  if (isnan(v)) return (uint8_t)(0x7F | sign);
  int top = fmt == O_E4M3 ? 0x7E : 0x7B;          /* largest finite magnitude code */
  if (a >= fmax) return (uint8_t)(top | sign);
  int lo = 0, hi = top;                            /* decode(lo) <= a < decode(hi) */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (o_fp8_decode((uint8_t)mid, fmt) <= a) lo = mid; else hi = mid;
  }
  double dlo = o_fp8_decode((uint8_t)lo, fmt), dhi = o_fp8_decode((uint8_t)(lo + 1), fmt);
  double q = (a - dlo) / (dhi - dlo);              /* exact: a has 24 bits, dhi - dlo = 2^k */
  int up = (double)r < ldexp(q, 32);
  return (uint8_t)((up ? lo + 1 : lo) | (int)sign);
}

/* Per-tensor cast with stochastic rounding: y[i] = sr(fl32(x[i] * s), word i)
 * and, when y_t is given, y_t[c][r] = y[r][c] (the same word per element). */
void o_cast_sr(const uint16_t* x, int64_t rows, int64_t cols, float s, int fmt, uint64_t seed,
               uint64_t offset, uint8_t* y, uint8_t* y_t) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      int64_t i = r * cols + c;
      float v = o_bf16_to_f32(x[i]) * s;
      uint8_t q = o_fp8_encode_sr(v, fmt, o_sr_word(seed, offset, (uint64_t)i));
      if (y) y[i] = q;
      if (y_t) y_t[c * rows + r] = q;
    }
}

/* ------------------------------------------------------------------ */
/* Exponentially weighted amax for delayed scaling.                    */
/* [MPG] "Delayed scaling (the default recipe)": the scale used at step */
/* t is the one right for step t-1, or an exponentially weighted        */
/* average of recent steps.  Reading: the average is taken of the amax  */
/* and the scale follows from it by the current-scaling rule:          */
/*   amax_new == 0 or non-finite: nothing changes;                      */
/*   ewma == 0 (no step seen yet): ewma = amax_new;                     */
/*   otherwise ewma = fl32(fl32(beta * ewma) + fl32(fl32(1 - beta) *    */
/*   amax_new));                                                        */
/*   then scale, scale_inv from ewma with the margin (kept on failure). */
/* ------------------------------------------------------------------ */
void o_amax_ewma_update(float* ewma, int64_t n, const float* amax_new, float beta, int fmt,
                        int margin, float* scale, float* scale_inv) {
  float omb = 1.0f - beta;
  for (int64_t i = 0; i < n; ++i) {
    float a = amax_new[i];
    if (!(a > 0.0f) || isinf(a)) continue;
    if (ewma[i] == 0.0f) {
      ewma[i] = a;
    } else {
      float t0 = beta * ewma[i];
      float t1 = omb * a;
      ewma[i] = t0 + t1;
    }
    float sc, si;
    if (o_compute_scale(ewma[i], fmt, margin, 0.0f, &sc, &si)) {
      scale[i] = sc;
      scale_inv[i] = si;
    }
  }
}

/* ------------------------------------------------------------------ */
/* bf16 rounding of a binary32 value (round to nearest even; a NaN     */
/* stays a quiet NaN).  Used to state the GEMM's BF16 output.          */
/* [MPG] "Mixed-precision accumulation": the FP32 accumulation is cast */
/* back to BF16 for the activation passed between layers.              */
/* ------------------------------------------------------------------ */
uint16_t o_f32_to_bf16(float f) {
  uint32_t b = b_of(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x0040u);
  b = b + 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

/* ------------------------------------------------------------------ */
/* Scaled FP8 GEMM oracles.                                            */
/*                                                                     */
/* D[m][n] = sum_k  dec(A[m][k]) * sa(m,k) * dec(B[n][k]) * sb(n,k)     */
/* with both operands K-contiguous (A [M][lda], B [N][ldb]), where the */
/* dequantisation scale of an operand is constant per tensor, per      */
/* (row, 128-wide K block) for 1x128 tiles, or per (128-row block,     */
/* 128-wide K block) for 128x128 blocks.  Scale arrays hold inverse    */
/* scales in the layouts of o_cast_block:                              */
/*   tensor   : s[0]                                                   */
/*   1x128    : s[kb * rows + row]                                     */
/*   128x128  : s[kb * ceil(rows/128) + row/128]                       */
/* [MPG] "Per-tensor scaling" (the matmul result is multiplied by the  */
/* inverse scales), "Skipping the BAcc accumulator promotion" and      */
/* "Mixed-precision accumulation" (partial products are accumulated in */
/* FP32), "Block-wise scaling at 128 granularity" (the block scales    */
/* are applied during the matmul).                                     */
/*                                                                     */
/* Every decoded E4M3 value is an integer times 2^-9 (|int| < 2^18),   */
/* every E5M2 value an integer times 2^-16 (|int| < 2^32), so a block  */
/* partial sum over 128 products is an exact integer S_kb times        */
/* 2^-(qa+qb).                                                         */
/*                                                                     */
/* Outputs, for every (m in ms) x (n in ns), row-major [nm][nn]:       */
/*   E : exact result (integer block sums, then the scales in long     */
/*       double; relative error ~2^-60);                               */
/*   F : the FP32-accumulated result: P_kb = fl32(S_kb * 2^-q),        */
/*       accumulated in increasing kb order in binary32;               */
/*       tensor mode: acc = fl32(acc + P_kb), then                     */
/*       fl32(fl32(acc * sa) * sb);                                    */
/*       block modes: acc = fl32(acc + fl32(P_kb * fl32(sa * sb)));    */
/*   Dm: sum_k |dec(a) sa * dec(b) sb| in double (the magnitude the    */
/*       error tolerances are scaled by).                              */
/* Any output pointer may be NULL.  Non-finite codes are not expected  */
/* (the encoder never emits Inf; NaN input codes give NaN).            */
/* ------------------------------------------------------------------ */
typedef struct {
  int64_t M, N, K, lda, ldb;
  const uint8_t* A; int a_fmt; int a_scaling; const float* a_sinv;
  const uint8_t* B; int b_fmt; int b_scaling; const float* b_sinv;
} o_gemm_args;

static float scale_at(int scaling, const float* s, int64_t rows, int64_t row, int64_t kb) {
  if (scaling == O_SCALE_TENSOR) return s[0];
  if (scaling == O_SCALE_ROW) return s[row];
  if (scaling == O_SCALE_1x128) return s[kb * rows + row];
  return s[kb * ((rows + 127) / 128) + row / 128];
}

/* integer significand of a decoded code: value = ival * 2^-q */
static int64_t fp8_int(uint8_t c, int fmt, int* is_nan) {
  double v = o_fp8_decode(c, fmt);
  if (isnan(v) || isinf(v)) { *is_nan = 1; return 0; }
  return (int64_t)ldexp(v, fmt == O_E4M3 ? 9 : 16);   /* exact */
}

typedef struct {
  const o_gemm_args* g;
  const int64_t* ms; int64_t nm;
  const int64_t* ns; int64_t nn;
  double* E; float* F; double* Dm;
  double* H; int hgroup; int hbits;   /* optional summation-precision bound */
  int64_t i0, i1;   /* range of ms indices for this worker */
} gemm_job;

/* floor(log2(v)) of a positive 128-bit integer */
static int ilog2_u128(unsigned __int128 v) {
  const uint64_t hi = (uint64_t)(v >> 64), lo = (uint64_t)v;
  if (hi) return 127 - __builtin_clzll(hi);
  return lo ? 63 - __builtin_clzll(lo) : -1;
}

static void* gemm_worker(void* p) {
  gemm_job* jb = (gemm_job*)p;
  const o_gemm_args* g = jb->g;
  /* per-tensor and per-row scales do not depend on the K block: the sum
   * over all of K is formed first and scaled once ([MPG] "Per-tensor
   * scaling": the matmul result is multiplied by the inverse scales;
   * "Per-row vs per-tensor scaling": one scale per row) */
  const int epi = (g->a_scaling == O_SCALE_TENSOR || g->a_scaling == O_SCALE_ROW) &&
                  (g->b_scaling == O_SCALE_TENSOR || g->b_scaling == O_SCALE_ROW);
  int64_t nkb = (g->K + 127) / 128;
  int qa = g->a_fmt == O_E4M3 ? 9 : 16, qb = g->b_fmt == O_E4M3 ? 9 : 16;
  int64_t* arow = (int64_t*)malloc(sizeof(int64_t) * (size_t)g->K);
  int64_t lut_b[256];
  int nan_b[256];
  /* decode table of B's format: integer significand of every code */
  for (int c = 0; c < 256; ++c) { nan_b[c] = 0; lut_b[c] = fp8_int((uint8_t)c, g->b_fmt, &nan_b[c]); }
  for (int64_t ii = jb->i0; ii < jb->i1; ++ii) {
    int64_t m = jb->ms[ii];
    int anan = 0;
    for (int64_t k = 0; k < g->K; ++k) arow[k] = fp8_int(g->A[m * g->lda + k], g->a_fmt, &anan);
    for (int64_t jj = 0; jj < jb->nn; ++jj) {
      int64_t n = jb->ns[jj];
      const uint8_t* brow = g->B + n * g->ldb;
      int bnan = 0;
      long double e_sum = 0.0L;
      double dsum = 0.0, hsum = 0.0;
      float acc = 0.0f;
      for (int64_t k = 0; k < g->K; ++k) bnan |= nan_b[brow[k]];
      for (int64_t kb = 0; kb < nkb; ++kb) {
        int64_t k0 = kb * 128, k1 = k0 + 128 < g->K ? k0 + 128 : g->K;
        __int128 S = 0;
        unsigned __int128 Sabs = 0;
        float sa = scale_at(g->a_scaling, g->a_sinv, g->M, m, kb);
        float sb = scale_at(g->b_scaling, g->b_sinv, g->N, n, kb);
        /* products of two integer significands (below 2^64 in magnitude;
         * both E5M2 may exceed 2^63), each formed once per block */
        __int128 pk[128];
        for (int64_t k = k0; k < k1; ++k) pk[k - k0] = (__int128)arow[k] * (__int128)lut_b[brow[k]];
        for (int64_t k = 0; k < k1 - k0; ++k) {
          S += pk[k];
          Sabs += (unsigned __int128)(pk[k] < 0 ? -pk[k] : pk[k]);
        }
        if (jb->H) {
          /* per group of hgroup consecutive k, with step q = 2^(e_max -
           * hbits) (e_max = exponent of the group's largest |product|):
           * a product that is not a multiple of q may lose less than q
           * (whichever way it is cut to the step); a multiple of q loses
           * nothing */
          for (int64_t k = 0; k < k1 - k0; k += jb->hgroup) {
            const int64_t ke = k + jb->hgroup < k1 - k0 ? k + jb->hgroup : k1 - k0;
            unsigned __int128 gm = 0;
            for (int64_t kk = k; kk < ke; ++kk) {
              unsigned __int128 ap = (unsigned __int128)(pk[kk] < 0 ? -pk[kk] : pk[kk]);
              if (ap > gm) gm = ap;
            }
            if (gm) {
              int e = ilog2_u128(gm) - jb->hbits;
              int inexact = 0;
              if (e > 0) {
                unsigned __int128 low = ((unsigned __int128)1 << e) - 1;
                for (int64_t kk = k; kk < ke; ++kk)
                  if ((unsigned __int128)(pk[kk] < 0 ? -pk[kk] : pk[kk]) & low) ++inexact;
              }
              hsum += (double)inexact * ldexp(1.0, e - (qa + qb)) * fabs((double)sa) * fabs((double)sb);
            }
          }
        }

        /* exact value of the block: S * 2^-(qa+qb) * sa * sb */
        long double Sl = (long double)S;               /* |S| < 2^65: exact to 2^-64 rel */
        long double blk = ldexpl(Sl, -(qa + qb));
        if (epi)
          e_sum += blk;                                  /* scales applied at the end */
        else
          e_sum += blk * (long double)sa * (long double)sb;
        dsum += ldexp((double)Sabs, -(qa + qb)) * fabs((double)sa) * fabs((double)sb);
        /* FP32-accumulated partner */
        {
          float P = ldexpf((float)S, -(qa + qb));      /* (float)S rounds once (RNE) */
          if (epi) {
            acc = acc + P;
          } else {
            float sab = sa * sb;
            float t = P * sab;
            acc = acc + t;
          }
        }
      }
      if (epi) {
        float sa = scale_at(g->a_scaling, g->a_sinv, g->M, m, 0);
        float sb = scale_at(g->b_scaling, g->b_sinv, g->N, n, 0);
        e_sum = e_sum * (long double)sa * (long double)sb;
        acc = acc * sa;
        acc = acc * sb;
      }
      if (anan || bnan) { e_sum = NAN; acc = NAN; dsum = NAN; }
      if (jb->E) jb->E[ii * jb->nn + jj] = (double)e_sum;
      if (jb->F) jb->F[ii * jb->nn + jj] = acc;
      if (jb->Dm) jb->Dm[ii * jb->nn + jj] = dsum;
      if (jb->H) jb->H[ii * jb->nn + jj] = hsum;
    }
  }
  free(arow);
  return NULL;
}

/* ldexpf on a float: exact for the power-of-two scalings used above
 * (results stay normal for |S| >= 1). */

void o_gemm_h(const o_gemm_args* g, const int64_t* ms, int64_t nm,
              const int64_t* ns, int64_t nn, double* E, float* F, double* Dm,
              double* H, int hgroup, int hbits, int nthreads);

void o_gemm(const o_gemm_args* g, const int64_t* ms, int64_t nm,
            const int64_t* ns, int64_t nn, double* E, float* F, double* Dm,
            int nthreads) {
  o_gemm_h(g, ms, nm, ns, nn, E, F, Dm, NULL, 8, 13, nthreads);
}

/* As o_gemm, plus H: a bound on the error of a matrix unit that sums each
 * group of `hgroup` consecutive products exactly after cutting every
 * product to a multiple of 2^(e_max - hbits) (e_max: exponent of the
 * group's largest product), toward zero or toward minus infinity: the
 * number of products that are not such multiples times that step, in
 * original (dequantised) units.  This is a tolerance model for tests of a
 * GPU implementation, not part of what the layer computes. */
void o_gemm_h(const o_gemm_args* g, const int64_t* ms, int64_t nm,
              const int64_t* ns, int64_t nn, double* E, float* F, double* Dm,
              double* H, int hgroup, int hbits, int nthreads) {
  pthread_t th[256];
  gemm_job jobs[256];
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > nm) nthreads = nm > 0 ? (int)nm : 1;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].g = g; jobs[t].ms = ms; jobs[t].nm = nm; jobs[t].ns = ns; jobs[t].nn = nn;
    jobs[t].E = E; jobs[t].F = F; jobs[t].Dm = Dm;
    jobs[t].H = H; jobs[t].hgroup = hgroup < 1 ? 1 : hgroup; jobs[t].hbits = hbits;
    jobs[t].i0 = nm * t / nthreads; jobs[t].i1 = nm * (t + 1) / nthreads;
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, gemm_worker, &jobs[t]);
  gemm_worker(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------ */
/* Unquantised reference R and its a-priori error bound.               */
/*                                                                     */
/* R[m][n] = sum_k a[m][k] * b[n][k] over the original bf16 operands,  */
/* in double.  The bound on |G - R| for a GEMM G of the quantised      */
/* operands follows from the format's unit roundoff u = 2^-(M+1), the  */
/* half subnormal spacing eta = 2^(emin-M-1) and saturation:           */
/*   per element  e_a = u_a'|a| + eta_a/s_a + sat_a,                    */
/*   u' = u (1+2^-24)^2 + 2^-22 (the binary32 multiply by s and the    */
/*        rounded inverse scale),                                      */
/*   sat_a = max(|a| - fmax/s_a, 0);                                   */
/*   |a^ b^ - a b| <= e_a (|b|(1+u_b') + eta_b/s_b) + |a| e_b;          */
/*   B = sum_k of that + gamma_{K+3} Dm + u_out |G|,                   */
/*   gamma_j = j 2^-23 / (1 - j 2^-23): binary32 summation in any      */
/*   order and with any rounding whose error stays below one ulp       */
/*   (FP8 x FP8 products are exact in binary32), plus the scale        */
/*   multiplies; u_out = 2^-8 for bf16 output, 0 for fp32 output.      */
/* The dequantised operand is dec(q) * s_inv with the stored inverse    */
/* scale, so a saturated element is off by |a| - fmax * s_inv; the      */
/* bound takes eta * s_inv * (1+2^-23) and fmax * s_inv / (1+2^-23)     */
/* (each rounded the safe way).                                        */
/* Inputs a, b are bf16 [M][K] and [N][K] (K-contiguous).              */
/* Outputs for (ms x ns): R (double) and Bnd (double, without the      */
/* u_out|G| term, which the caller adds from its own G).               */
/* ------------------------------------------------------------------ */
typedef struct {
  const o_gemm_args* g;
  const uint16_t* a; const uint16_t* b;
  const int64_t* ms; int64_t nm; const int64_t* ns; int64_t nn;
  double* R; double* Bnd; int64_t i0, i1;
} ref_job;

static void fmt_consts(int fmt, double* u, double* eta) {
  if (fmt == O_E4M3) { *u = ldexp(1.0, -4); *eta = ldexp(1.0, -10); }
  else               { *u = ldexp(1.0, -3); *eta = ldexp(1.0, -17); }
}

static void* ref_worker(void* p) {
  ref_job* jb = (ref_job*)p;
  const o_gemm_args* g = jb->g;
  double ua, ea, ub, eb;
  double infl = (1.0 + ldexp(1.0, -24)) * (1.0 + ldexp(1.0, -24));
  double up = 1.0 + ldexp(1.0, -23);
  double fa = o_fp8_max(g->a_fmt), fb = o_fp8_max(g->b_fmt);
  double gam = (double)(g->K + 3) * ldexp(1.0, -23);
  gam = gam / (1.0 - gam);
  fmt_consts(g->a_fmt, &ua, &ea);
  fmt_consts(g->b_fmt, &ub, &eb);
  ua = ua * infl + ldexp(1.0, -22);
  ub = ub * infl + ldexp(1.0, -22);
  for (int64_t ii = jb->i0; ii < jb->i1; ++ii) {
    int64_t m = jb->ms[ii];
    for (int64_t jj = 0; jj < jb->nn; ++jj) {
      int64_t n = jb->ns[jj];
      double r = 0.0, bnd = 0.0, dm = 0.0;
      for (int64_t k = 0; k < g->K; ++k) {
        int64_t kb = k / 128;
        double av = (double)o_bf16_to_f32(jb->a[m * g->K + k]);
        double bv = (double)o_bf16_to_f32(jb->b[n * g->K + k]);
        double sia0 = (double)scale_at(g->a_scaling, g->a_sinv, g->M, m, kb);
        double sib0 = (double)scale_at(g->b_scaling, g->b_sinv, g->N, n, kb);
        double sia = sia0 * up, sib = sib0 * up;
        double sata = fabs(av) - fa * sia0 / up; if (sata < 0) sata = 0;
        double satb = fabs(bv) - fb * sib0 / up; if (satb < 0) satb = 0;
        double e_a = ua * fabs(av) + ea * sia + sata;
        double e_b = ub * fabs(bv) + eb * sib + satb;
        double bhat = fabs(bv) * (1.0 + ub) + eb * sib;
        double ahat = fabs(av) * (1.0 + ua) + ea * sia;
        r += av * bv;
        bnd += e_a * bhat + fabs(av) * e_b;
        dm += ahat * bhat;
      }
      jb->R[ii * jb->nn + jj] = r;
      jb->Bnd[ii * jb->nn + jj] = bnd + gam * dm;
    }
  }
  return NULL;
}

void o_gemm_ref_bound(const o_gemm_args* g, const uint16_t* a_bf16, const uint16_t* b_bf16,
                      const int64_t* ms, int64_t nm, const int64_t* ns, int64_t nn,
                      double* R, double* Bnd, int nthreads) {
  pthread_t th[256];
  ref_job jobs[256];
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > nm) nthreads = nm > 0 ? (int)nm : 1;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].g = g; jobs[t].a = a_bf16; jobs[t].b = b_bf16;
    jobs[t].ms = ms; jobs[t].nm = nm; jobs[t].ns = ns; jobs[t].nn = nn;
    jobs[t].R = R; jobs[t].Bnd = Bnd;
    jobs[t].i0 = nm * t / nthreads; jobs[t].i1 = nm * (t + 1) / nthreads;
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, ref_worker, &jobs[t]);
  ref_worker(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------ */
/* Array helpers for the Python test harness.                          */
/* ------------------------------------------------------------------ */
void o_encode_array(const float* x, int64_t n, int fmt, uint8_t* y) {
  for (int64_t i = 0; i < n; ++i) y[i] = o_fp8_encode(x[i], fmt);
}

void o_decode_array(const uint8_t* c, int64_t n, int fmt, double* v) {
  for (int64_t i = 0; i < n; ++i) v[i] = o_fp8_decode(c[i], fmt);
}

void o_f32_to_bf16_array(const float* x, int64_t n, uint16_t* y) {
  for (int64_t i = 0; i < n; ++i) y[i] = o_f32_to_bf16(x[i]);
}
