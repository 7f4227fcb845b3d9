/*
 * fp8lin.h -- C ABI of the FP8 scaled linear layer for AMD gfx950 (CDNA4).
 *
 * The layer: an amax reduction, a scale (current per-tensor, delayed from an
 * amax history, or block-wise), a saturating round-to-nearest-even cast to
 * FP8 (E4M3 for activations and weights, E5M2 for gradients), and the
 * forward / dgrad / wgrad GEMMs with FP32 accumulation and the inverse
 * scales applied in the epilogue (per-tensor) or per 128-wide K block
 * (block-wise).
 *
 * Sources, cited by page title and section:
 *   [MPG]  "Mixed Precision LLM Training: The Complete Guide"
 *   [TALK] PyData Amsterdam 2026, "FP8 for pretraining" (talk abstract)
 *   [P3]   "Training and inference of large language models using 8-bit
 *          floating point" (arXiv 2309.17224 library entry: abstract and
 *          reviews)
 *
 * Conventions for every entry point:
 *   - Pointers are caller-owned DEVICE memory on the current HIP device,
 *     unless stated otherwise.  The library never allocates, frees or keeps
 *     a pointer after the call returns.
 *   - Every call only enqueues work on `stream` (0 = the null stream) and
 *     returns; nothing is read back to the host, so a sequence of calls can
 *     run without host synchronisation.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     any error code other than FP8_ERR_LAUNCH nothing was enqueued.
 *   - bf16 tensors are row-major [rows][cols] arrays of 16-bit patterns.
 *   - Outputs named *amax* are overwritten (not max-accumulated).
 *   - No global mutable state: calls on different streams may interleave.
 *   - FP8 codes are OCP E4M3 (max 448, no Inf, NaN = 0x7F/0xFF) and OCP E5M2
 *     (max 57344); the cast saturates finite overflow and +-Inf to +-max,
 *     maps NaN to 0x7F|sign, keeps the sign of zero, and rounds to nearest
 *     even after a binary32 multiply by the scale.
 */
#ifndef FP8LIN_H
#define FP8LIN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8LIN_ABI_VERSION 10

/* [MPG] "The precision formats", "FP8 E4M3", "FP8 E5M2": E4M3 = 4 exponent
 * and 3 mantissa bits, range about 2^-9..448; E5M2 = 5 and 2, range about
 * 2^-16..57344.  "The HYBRID recipe": E4M3 forward, E5M2 for gradients. */
typedef enum { FP8_E4M3 = 0, FP8_E5M2 = 1 } fp8_format;

typedef enum {
  FP8_OK = 0,
  FP8_ERR_NULL = 1,         /* a required pointer is NULL */
  FP8_ERR_SHAPE = 2,        /* negative size, or a shape rule is broken */
  FP8_ERR_ALIGN = 3,        /* pointer or leading dimension misaligned */
  FP8_ERR_UNSUPPORTED = 4,  /* valid request the library does not implement */
  FP8_ERR_LAUNCH = 5,       /* the HIP runtime rejected a kernel launch */
  FP8_ERR_ARG = 6           /* an enum or scalar argument is out of range */
} fp8_status;

/* [MPG] "Calibration deep dive > Dynamic calibration (delayed scaling)":
 * amax_compute_algo "max" (over the history) or "most_recent". */
typedef enum { FP8_AMAX_MAX = 0, FP8_AMAX_MOST_RECENT = 1 } fp8_amax_algo;

/* [MPG] "Per-row vs per-tensor scaling" and "DeepSeek FP8 training recipe
 * in detail > Block-wise scaling at 128 granularity": one scale per tensor,
 * per 128-element segment of a row (1x128), or per 128x128 block.
 * The *_POW2 codes (GEMM operands only) are the same block layouts whose
 * inverse scales are exact powers of two 2^e, |e| <= 126, as produced by
 * fp8_cast_block_pow2 ([P3] exponent-bias scaling).
 * FP8_SCALE_ROW (GEMM operands only): one scale per row of a K-contiguous
 * operand, i.e. per token or per output channel, as produced by
 * fp8_cast_rowwise ("Per-row vs per-tensor scaling"). */
typedef enum {
  FP8_SCALE_TENSOR = 0,
  FP8_SCALE_1x128 = 1,
  FP8_SCALE_128x128 = 2,
  FP8_SCALE_1x128_POW2 = 3,
  FP8_SCALE_128x128_POW2 = 4,
  FP8_SCALE_ROW = 5
} fp8_scaling;

/* GEMM output: BF16, FP32, or FP8 codes quantised in the epilogue (the
 * next layer's cast fused into this GEMM). */
typedef enum { FP8_OUT_BF16 = 0, FP8_OUT_F32 = 1, FP8_OUT_E4M3 = 2, FP8_OUT_E5M2 = 3 } fp8_out_dtype;

/* ABI version (FP8LIN_ABI_VERSION of the built library). */
int fp8_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fp8_status_string(fp8_status status);

/* ------------------------------------------------------------------------
 * fp8_amax -- amax = max |x| over a bf16 tensor.
 * [MPG] "Transformer Engine internals > Per-tensor scaling": the scale is
 * set from the tensor's maximum absolute value.
 *   x_bf16  [rows][ld] bf16 (the first cols of each row are read),
 *           16-byte aligned; ld >= cols, in elements (ld == cols: a
 *           contiguous tensor).
 *   amax    1 float, overwritten.  The maximum is exact (no rounding is
 *           involved); a NaN element makes the result NaN; an empty tensor
 *           gives 0.
 * Errors: FP8_ERR_NULL (x with rows*cols > 0, or amax NULL), FP8_ERR_SHAPE
 * (negative size, ld < cols), FP8_ERR_ALIGN (x not 16-byte aligned).
 * ---------------------------------------------------------------------- */
fp8_status fp8_amax(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld, float* amax,
                    hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_cast_stats -- saturation and underflow counts of the per-tensor cast
 * (fp8_cast_e4m3 / e5m2 with the same scale), for the diagnostic
 * dashboard's overflow and underflow ratios per layer.
 * [MPG] "Numerical-failure taxonomy > A diagnostic dashboard".
 * With v = fl32(x * scale[0]) as the cast computes it:
 *   counts[0] += number of elements with |v| beyond the format's largest
 *                finite value (448 / 57344; +-Inf included, NaN not);
 *   counts[1] += number of nonzero elements x whose code is +-0 (|v| at
 *                most half the smallest subnormal step: 2^-10 / 2^-17).
 *   x_bf16  [rows][cols] bf16, contiguous, 16-byte aligned.
 *   scale   1 float (device).
 *   counts  2 uint64 (device), 8-byte aligned; added to, never cleared.
 * Reads x once (2 B/elem); writes nothing else.
 * Errors: FP8_ERR_NULL (counts; x or scale with rows*cols > 0),
 * FP8_ERR_SHAPE, FP8_ERR_ALIGN, FP8_ERR_ARG (fmt).
 * ---------------------------------------------------------------------- */
fp8_status fp8_cast_stats(const void* x_bf16, int64_t rows, int64_t cols, fp8_format fmt,
                          const float* scale, uint64_t* counts, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_amax_acc -- fp8_amax with the result max-accumulated into *amax_acc
 * instead of overwriting it: one kernel, no fill ahead of it.
 * [MPG] "Delayed scaling (the default recipe)": the step's amax goes into
 * the tensor's history slot, which fp8_amax_history_update_reset clears
 * after reading it, so the next step accumulates into zero.
 *   amax_acc  1 float (device), required: on return max(old value, max |x|)
 *             (as binary32 bit patterns of |value|: a NaN element makes it
 *             NaN).  Calls that accumulate into one slot may overlap.
 * Other arguments and errors as fp8_amax.
 * ---------------------------------------------------------------------- */
fp8_status fp8_amax_acc(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld,
                        float* amax_acc, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_compute_scale -- current scaling: scale = fl32(fmax / amax) * 2^-margin,
 * scale_inv = fl32(1 / scale), elementwise over n tensors.
 * [MPG] "Per-tensor scaling" (the scale puts the amax at the top of the FP8
 * range; the matmul result is multiplied by the inverse scale) and the
 * DelayedScaling recipe's `margin` argument (formula not given; read as a
 * division of the scale by 2^margin).
 *   amax       [n] floats (device).
 *   fmt        fmax = 448 (E4M3) or 57344 (E5M2).
 *   margin     0..64.
 *   scale, scale_inv  [n] floats, overwritten.
 * amax == 0 or non-finite: scale = 1, scale_inv = 1 ([MPG] "torch.compile
 * and FP8": no scale update for an all-zero tensor).  A quotient that
 * overflows binary32 is clamped to FLT_MAX.  Divisions are correctly
 * rounded.
 * Errors: FP8_ERR_NULL, FP8_ERR_SHAPE (n < 0), FP8_ERR_ARG (fmt, margin).
 * ---------------------------------------------------------------------- */
fp8_status fp8_compute_scale(const float* amax, int64_t n, fp8_format fmt, int margin,
                             float* scale, float* scale_inv, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_compute_scale_pow2 -- current scaling with power-of-two scales.
 * [P3] abstract and reviews: the scale is an exponent bias chosen from the
 * tensor's maximum (FP8-AMAX), matching its range to the format's; the
 * page does not print the formula.  Reading: scale = 2^e with e the largest
 * integer such that amax * 2^e <= fmax (the amax lands in (fmax/2, fmax],
 * nothing saturates), then e -= margin, e clamped to [-126, 126];
 * scale_inv = 2^-e.  Both are exact, so dequantisation is exact.
 * Arguments, fallback rule and errors as fp8_compute_scale.
 * ---------------------------------------------------------------------- */
fp8_status fp8_compute_scale_pow2(const float* amax, int64_t n, fp8_format fmt, int margin,
                                  float* scale, float* scale_inv, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_amax_history_update -- delayed scaling from an amax history.
 * [MPG] "Delayed scaling (the default recipe)" and "History-based scaling":
 * the scale used at step t+1 comes from the maxima of the last `len` steps.
 * For each tensor i < n:
 *   history[i][len-1..1] = history[i][len-2..0]; history[i][0] = amax_new[i];
 *   eff = max_j history[i][j] (FP8_AMAX_MAX; NaN propagates) or
 *         history[i][0] (FP8_AMAX_MOST_RECENT);
 *   if eff > 0 and finite: scale[i] = fl32(fmax/eff)*2^-margin,
 *                          scale_inv[i] = fl32(1/scale[i]);
 *   otherwise scale[i], scale_inv[i] keep their previous values.
 *   history    [n][len] floats, newest first, updated in place (initialise
 *              to 0 with scale = scale_inv = 1 before the first step).
 *   amax_new   [n] floats (e.g. the fused amax of the step's casts).
 * Stream order makes the update happen after the step's casts and GEMMs
 * that read the old scale when all are enqueued on one stream.
 * Errors: FP8_ERR_NULL, FP8_ERR_SHAPE (n < 0, len < 1 or > 1024),
 * FP8_ERR_ARG (fmt, margin, algo).
 * ---------------------------------------------------------------------- */
fp8_status fp8_amax_history_update(float* history, int64_t n, int64_t len,
                                   const float* amax_new, fp8_format fmt, int margin,
                                   fp8_amax_algo algo, float* scale, float* scale_inv,
                                   hipStream_t stream);

/* fp8_amax_history_update_pow2 -- the same update with the power-of-two
 * scale of fp8_compute_scale_pow2 ([P3] exponent bias) from the effective
 * amax; arguments and errors as fp8_amax_history_update. */
fp8_status fp8_amax_history_update_pow2(float* history, int64_t n, int64_t len,
                                        const float* amax_new, fp8_format fmt, int margin,
                                        fp8_amax_algo algo, float* scale, float* scale_inv,
                                        hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_amax_history_update_reset -- fp8_amax_history_update, after which
 * every consumed amax_new[i] is set to 0.
 * [MPG] "Delayed scaling (the default recipe)": the amax observed at step t
 * enters the history that sets the scale of step t+1.  With the slots
 * cleared here, the casts of the next step accumulate into them with
 * fp8_cast_amax_acc and no separate zeroing is needed between steps: one
 * step is then casts -> GEMMs -> this update, with amax_new starting at 0.
 *   amax_new   [n] floats (device), read, then overwritten with 0.
 *   Other arguments, order and errors as fp8_amax_history_update.
 * ---------------------------------------------------------------------- */
fp8_status fp8_amax_history_update_reset(float* history, int64_t n, int64_t len, float* amax_new,
                                         fp8_format fmt, int margin, fp8_amax_algo algo,
                                         float* scale, float* scale_inv, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_amax_ewma_update -- delayed scaling from an exponentially weighted
 * amax.  [MPG] "Delayed scaling (the default recipe)": the scale used at
 * step t is the one right for step t-1, or an exponentially weighted
 * average of recent steps (read as an average of the amax, from which the
 * scale follows).  For each tensor i < n, with a = amax_new[i]:
 *   a == 0 or non-finite: nothing changes;
 *   ewma[i] == 0 (no step seen yet): ewma[i] = a;
 *   else ewma[i] = fl32(fl32(beta * ewma[i]) + fl32(fl32(1 - beta) * a));
 *   then scale[i] = fl32(fmax / ewma[i]) * 2^-margin, scale_inv[i] =
 *   fl32(1 / scale[i]) (overflow clamped to FLT_MAX).
 *   ewma       [n] floats, in place (initialise to 0, scale = scale_inv = 1).
 *   beta       weight of the past, 0 <= beta <= 1 (0: the newest amax).
 * Errors: FP8_ERR_NULL, FP8_ERR_SHAPE (n < 0), FP8_ERR_ALIGN, FP8_ERR_ARG
 * (fmt, margin outside 0..64, beta outside [0, 1] or NaN).
 * ---------------------------------------------------------------------- */
fp8_status fp8_amax_ewma_update(float* ewma, int64_t n, const float* amax_new, float beta,
                                fp8_format fmt, int margin, float* scale, float* scale_inv,
                                hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_cast_e4m3 / fp8_cast_e5m2 -- per-tensor saturating RNE cast,
 * q = encode(fl32(x * scale)), with optional fused transpose and amax.
 * [MPG] "Per-tensor scaling" (multiply by the scale before quantising);
 * [TALK] outline 05:00-15:00 (E4M3 for activations and weights, E5M2 for
 * gradients).
 *   x_bf16    [rows][cols] bf16, 16-byte aligned.
 *   scale     1 float (device): the quantisation scale (not the inverse).
 *   y         [rows][cols] FP8 codes, or NULL.
 *   y_t       [cols][rows] FP8 codes (y_t[c][r] = y[r][c]), or NULL.
 *   amax_out  1 float, overwritten with max |x| (as fp8_amax), or NULL.
 *   y and y_t must not both be NULL (unless the tensor is empty); y, y_t
 *   16-byte aligned.
 * Errors: FP8_ERR_NULL, FP8_ERR_SHAPE, FP8_ERR_ALIGN.
 * ---------------------------------------------------------------------- */
fp8_status fp8_cast_e4m3(const void* x_bf16, int64_t rows, int64_t cols, const float* scale,
                         uint8_t* y, uint8_t* y_t, float* amax_out, hipStream_t stream);
fp8_status fp8_cast_e5m2(const void* x_bf16, int64_t rows, int64_t cols, const float* scale,
                         uint8_t* y, uint8_t* y_t, float* amax_out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_cast_amax_acc -- the per-tensor cast of fp8_cast_e4m3 / e5m2 with the
 * fused amax max-accumulated into *amax_acc instead of overwriting it.
 * [MPG] "Per-tensor scaling" (the cast), "Delayed scaling (the default
 * recipe)" (the amax of the step feeds the next step's scale): with the
 * slot cleared by fp8_amax_history_update_reset, a delayed-scaling step
 * needs no zeroing kernel before its casts.
 *   fmt        FP8_E4M3 or FP8_E5M2.
 *   amax_acc   1 float (device), required: on return
 *              max(previous value, max |x|), compared as binary32 bit
 *              patterns, so the previous value must be +0 or positive
 *              (NaN in x propagates as in fp8_amax).
 *   Other arguments, layouts and errors as fp8_cast_e4m3, plus FP8_ERR_ARG
 *   (fmt) and FP8_ERR_NULL (amax_acc).  Calls that accumulate into one slot
 *   may run concurrently on several streams.
 * ---------------------------------------------------------------------- */
fp8_status fp8_cast_amax_acc(const void* x_bf16, int64_t rows, int64_t cols, fp8_format fmt,
                             const float* scale, uint8_t* y, uint8_t* y_t, float* amax_acc,
                             hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_cast_sr -- per-tensor cast with stochastic rounding.
 * [MPG] "Stochastic rounding": round up or down at random according to the
 * remainder, which keeps the rounded value unbiased (used for gradients);
 * [TALK] outline: "rounding techniques".
 * With v = fl32(x * scale) and lo <= |v| < hi the two neighbouring FP8
 * magnitudes, the code is hi when r < (|v| - lo) / (hi - lo) * 2^32, else
 * lo (sign kept), where r is the element's random word; |v| >= fmax and
 * +-Inf saturate to +-fmax, NaN gives 0x7F | sign.  The word of element i
 * (row-major index) is word i % 4 of Philox4x32-10 (Salmon et al., SC 2011)
 * with counter (i / 4 low, i / 4 high, offset low, offset high) and key
 * (seed low, seed high); y_t holds the same codes transposed.  Calls with the
 * same (seed, offset) repeat the same draw; a call with another offset draws
 * fresh words (the offset is its own pair of counter words).  The values are
 * baked into a captured graph: see fp8_cast_sr_state.
 *   fmt        FP8_E4M3 or FP8_E5M2.
 *   Other arguments, layouts and errors as fp8_cast_e4m3, plus FP8_ERR_ARG
 *   (fmt).
 * ---------------------------------------------------------------------- */
fp8_status fp8_cast_sr(const void* x_bf16, int64_t rows, int64_t cols, fp8_format fmt,
                       const float* scale, uint64_t seed, uint64_t offset, uint8_t* y,
                       uint8_t* y_t, float* amax_out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_cast_sr_state -- fp8_cast_sr with the generator state in device
 * memory, for steps captured once and replayed.  [MPG] "Stochastic
 * rounding": the rounding is unbiased only if every step draws fresh random
 * words, which by-value (seed, offset) cannot give a replayed graph.
 *   rng_state  2 x uint64 (device, 8-byte aligned, caller-owned): seed and
 *              offset, read by the cast when it runs on the stream; the codes
 *              equal fp8_cast_sr with those values.  Afterwards, in stream
 *              order, rng_state[1] += advance (modulo 2^64).
 *   advance    any nonzero value gives the next call fresh words: the offset
 *              is its own pair of Philox counter words, distinct from the
 *              element index; 0 repeats the draw.
 *   Other arguments, layouts and errors as fp8_cast_sr, plus FP8_ERR_NULL
 *   (rng_state) and FP8_ERR_ALIGN (rng_state not 8-byte aligned).  Calls on
 *   one rng_state must be stream-ordered (concurrent calls race on it).
 * ---------------------------------------------------------------------- */
fp8_status fp8_cast_sr_state(const void* x_bf16, int64_t rows, int64_t cols, fp8_format fmt,
                             const float* scale, uint64_t* rng_state, uint64_t advance,
                             uint8_t* y, uint8_t* y_t, float* amax_out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_cast_block -- block-wise cast with per-tile scales computed on the fly.
 * [MPG] "DeepSeek FP8 training recipe in detail > Block-wise scaling at 128
 * granularity": one scale per 128x128 weight block, one per 128-element
 * activation segment, stored next to the data and applied in the matmul.
 * Per tile: amax over the elements present, scale = fl32(fmax/amax)
 * (1 for an all-zero or non-finite tile), scale_inv = fl32(1/scale), then
 * the cast of fp8_cast_e4m3 with that scale.
 *   x_bf16   [rows][cols] bf16, 16-byte aligned.
 *   tile == FP8_SCALE_1x128:
 *     y         [rows][cols], tiles of 128 consecutive columns in one row;
 *     scale_inv [ceil(cols/128)][rows]  (kb-major);
 *     y_t       [cols][rows], tiles of 128 consecutive ROWS in one column
 *               (the token-axis tiles of the transposed operand), each
 *               quantised from bf16 with its own scale;
 *     scale_inv_t [ceil(rows/128)][cols].
 *   tile == FP8_SCALE_128x128:
 *     one scale per 128x128 block; y_t is the byte transpose of y;
 *     scale_inv   [ceil(cols/128)][ceil(rows/128)];
 *     scale_inv_t [ceil(rows/128)][ceil(cols/128)] (same values, transposed).
 *   Each of (y, scale_inv) and (y_t, scale_inv_t) is either both given or
 *   both NULL, and at least one pair is given (an empty tensor needs no
 *   pointers and enqueues nothing).  y, y_t 16-byte aligned.
 * Errors: FP8_ERR_NULL, FP8_ERR_SHAPE, FP8_ERR_ALIGN, FP8_ERR_ARG.
 * ---------------------------------------------------------------------- */
fp8_status fp8_cast_block(const void* x_bf16, int64_t rows, int64_t cols, fp8_format fmt,
                          fp8_scaling tile, uint8_t* y, float* scale_inv, uint8_t* y_t,
                          float* scale_inv_t, hipStream_t stream);

/* fp8_cast_block_pow2 -- fp8_cast_block with power-of-two tile scales (the
 * rule of fp8_compute_scale_pow2 on each tile's amax, margin 0; [P3]
 * exponent bias applied per DeepSeek-style block).  The scales it writes
 * are valid FP8_SCALE_1x128_POW2 / FP8_SCALE_128x128_POW2 GEMM operands.
 * Arguments (tile is FP8_SCALE_1x128 or FP8_SCALE_128x128) and errors as
 * fp8_cast_block. */
fp8_status fp8_cast_block_pow2(const void* x_bf16, int64_t rows, int64_t cols, fp8_format fmt,
                               fp8_scaling tile, uint8_t* y, float* scale_inv, uint8_t* y_t,
                               float* scale_inv_t, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_cast_rowwise -- row-wise (per-channel) cast with scales computed on
 * the fly.  [MPG] "Per-row vs per-tensor scaling": one scale per row of the
 * matrix rather than one per tensor, so an outlier row or column only
 * coarsens its own scale (torchao's row-wise recipe).
 *   x_bf16       [rows][cols] bf16, 16-byte aligned.
 *   y            [rows][cols]: row r quantised with s_r = fl32(fmax / amax_r),
 *                amax_r = max_c |x[r][c]| (s_r = 1 for an all-zero or
 *                non-finite row), codes as fp8_cast_e4m3 / e5m2;
 *   scale_inv    [rows]: fl32(1 / s_r)  (an FP8_SCALE_ROW GEMM operand);
 *   y_t          [cols][rows]: y_t[c][r] quantised with the scale of column
 *                c, s_c = fl32(fmax / max_r |x[r][c]|) (same fallback) -- the
 *                K-contiguous operand of the GEMMs that reduce over rows;
 *   scale_inv_t  [cols]: fl32(1 / s_c).
 *   Each of (y, scale_inv) and (y_t, scale_inv_t) is either both given or
 *   both NULL, and at least one pair is given (an empty tensor needs no
 *   pointers and enqueues nothing).  y, y_t 16-byte aligned.  The memory
 *   of y_t and scale_inv_t also serves as workspace while the call runs
 *   (column maxima); both hold their final values once the call's work
 *   has completed in stream order.
 * Errors: FP8_ERR_NULL, FP8_ERR_SHAPE, FP8_ERR_ALIGN, FP8_ERR_ARG (fmt).
 * ---------------------------------------------------------------------- */
fp8_status fp8_cast_rowwise(const void* x_bf16, int64_t rows, int64_t cols, fp8_format fmt,
                            uint8_t* y, float* scale_inv, uint8_t* y_t, float* scale_inv_t,
                            hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_scaled_gemm -- D[m][n] = sum_k A[m][k] * B[n][k] with FP8 operands,
 * FP32 accumulation and dequantisation.
 * [MPG] "Per-tensor scaling" (multiply the matmul result by the inverse
 * scales), "Skipping the BAcc accumulator promotion" and "Mixed-precision
 * accumulation" (partial products accumulate in FP32; the result is cast to
 * BF16), "Block-wise scaling at 128 granularity" (block scales applied
 * during the matmul).
 * Both operands are K-contiguous ("TN"): A [M][lda], B [N][ldb] FP8 codes.
 * The layer's three GEMMs are operand choices (weights stored [in][out]):
 *   forward  Y  = X W      : A = X_q   [T][in],  B = W^T_q  [out][in]
 *   dgrad    dX = dY W^T   : A = dY_q  [T][out], B = W_q    [in][out]
 *   wgrad    dW = X^T dY   : A = X^T_q [in][T],  B = dY^T_q [out][T]
 * Inverse-scale layouts (as produced by the casts):
 *   FP8_SCALE_TENSOR  : 1 float;
 *   FP8_SCALE_1x128   : [ceil(K/128)][rows]       (rows = M for A, N for B);
 *   FP8_SCALE_128x128 : [ceil(K/128)][ceil(rows/128)];
 *   FP8_SCALE_1x128_POW2, FP8_SCALE_128x128_POW2: the same layouts, every
 *   value an exact power of two 2^e with |e| <= 126 (fp8_cast_block_pow2);
 *   other values give unspecified (memory-safe) results.  When every
 *   block-scaled operand is a *_POW2 one, the block scales are applied
 *   inside the matrix instruction (exact power-of-two scaling of each
 *   128-wide K block) and a per-tensor operand's scale in the epilogue;
 *   mixed with a plain block operand, all block scales are promoted in
 *   FP32 as for FP8_SCALE_1x128 / FP8_SCALE_128x128;
 *   FP8_SCALE_ROW     : [rows] (one per row of the operand; combines with
 *   FP8_SCALE_TENSOR or FP8_SCALE_ROW only, else FP8_ERR_UNSUPPORTED).
 * Result: tensor or row x tensor or row: D = ((sum_k a b) * sa(m)) * sb(n),
 * one FP32 sum over all of K scaled in the epilogue; any block scaling:
 * D = sum_kb (sum_{k in kb} a b) * sa(m,kb) * sb(n,kb), each 128-wide K
 * block promoted into the FP32 accumulator.  D is [M][ldd], BF16 (round
 * to nearest even) or FP32.  accumulate = 1 (FP32 output only) adds the
 * result to the existing D.  d_amax (nullable, 1 float) is overwritten with
 * max |D| of the stored output values (a one-word fill runs ahead of the
 * GEMM on the stream), or, with amax_accumulate = 1, max-accumulated into
 * the value already there (no fill: the caller owns the slot, e.g. one
 * cleared by fp8_amax_history_update_reset; calls that accumulate into one
 * slot may overlap).
 * FP8 output (d_dtype FP8_OUT_E4M3 / FP8_OUT_E5M2; [TALK] outline
 * "quantisation fusions"; [MPG] "Transformer Engine internals": the cast
 * that the next layer would do, fused into this GEMM's epilogue): with v the
 * FP32 result above (before any BF16 rounding), D[m][n] = encode(fl32(v *
 * d_scale[0])) as in fp8_cast_e4m3 / e5m2; D_t (nullable) [N][ldt] receives
 * the same codes transposed (the next layer's wgrad operand); d_amax is
 * max |v| (the amax of the quantised tensor, for its delayed scaling).
 * accumulate must be 0; requires ldt >= M when D_t is given.
 * amax_accumulate: 0 or 1 (FP8_ERR_ARG otherwise), see d_amax.
 * Shape rules: M, N, K >= 0; K % 16 == 0 (tensor and row modes) or
 * K % 128 == 0 (block modes); lda, ldb >= K and multiples of 16; ldd >= N; A, B 16-byte
 * aligned; D 4-byte aligned.  K == 0 gives D = 0 (or D unchanged when
 * accumulating).
 * Errors: FP8_ERR_NULL, FP8_ERR_SHAPE, FP8_ERR_ALIGN, FP8_ERR_ARG (also
 * D_t with a non-FP8 output), FP8_ERR_UNSUPPORTED (accumulate with a BF16
 * or FP8 output; FP8 output with lda or ldb beyond the large-tile kernel's
 * 32-bit panel offsets, i.e. 256 * ld >= 2^31; FP8_SCALE_ROW with a block
 * operand).
 * ---------------------------------------------------------------------- */
typedef struct {
  int64_t M, N, K;
  int64_t lda, ldb, ldd;
  const uint8_t* A; fp8_format a_fmt; fp8_scaling a_scaling; const float* a_scale_inv;
  const uint8_t* B; fp8_format b_fmt; fp8_scaling b_scaling; const float* b_scale_inv;
  void* D; fp8_out_dtype d_dtype;
  float* d_amax;
  int accumulate;
  const float* d_scale;   /* FP8 output: quantisation scale (1 float); else ignored */
  uint8_t* D_t;           /* FP8 output: transposed codes [N][ldt], or NULL */
  int64_t ldt;
  int amax_accumulate;    /* 1: max-accumulate into *d_amax instead of overwriting */
} fp8_gemm_args;

fp8_status fp8_scaled_gemm(const fp8_gemm_args* args, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8LIN_H */
