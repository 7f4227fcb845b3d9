/*
 * fp8_brute.c -- brute-force nearest-value FP8 encoder, used only to pin the
 * bit-manipulation encoder of fp8_oracle.c (TEST INFRASTRUCTURE ONLY).
 *
 * It follows the definition of round-to-nearest-even with saturation as a
 * search, not as bit arithmetic: among all finite FP8 values pick the one
 * nearest to |x|; on an exact tie pick the code whose mantissa LSB (the code
 * LSB) is 0; values past the largest finite value therefore land on it;
 * NaN maps to 0x7F | sign and the sign is always kept.
 * ("Mixed Precision LLM Training: The Complete Guide", "The precision
 * formats" table: E4M3 and E5M2 field widths and ranges.)
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

double o_fp8_decode(uint8_t c, int fmt);
uint8_t o_fp8_encode(float x, int fmt);

typedef struct { double v[128]; int n; } table_t;

/* non-negative finite codes 0 .. n-1 in increasing value order */
static void build_table(int fmt, table_t* t) {
  t->n = 0;
  for (int c = 0; c < 128; ++c) {
    double v = o_fp8_decode((uint8_t)c, fmt);
    if (isnan(v) || isinf(v)) break;
    t->v[t->n++] = v;
  }
}

static uint8_t brute_encode(const table_t* t, float x) {
  uint32_t u; memcpy(&u, &x, 4);
  uint8_t sign = (uint8_t)((u >> 31) << 7);
  double a;
  int lo, hi;
  if (isnan(x)) return (uint8_t)(sign | 0x7F);
  a = fabs((double)x);
  if (a >= t->v[t->n - 1]) return (uint8_t)(sign | (t->n - 1));
  /* largest code with value <= a (binary search on the sorted table) */
  lo = 0; hi = t->n - 1;
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (t->v[mid] <= a) lo = mid; else hi = mid;
  }
  /* a in [v[lo], v[lo+1]): compare 2a with v[lo] + v[lo+1] (all exact) */
  {
    double two_a = 2.0 * a, sum = t->v[lo] + t->v[lo + 1];
    int pick;
    if (two_a < sum) pick = lo;
    else if (two_a > sum) pick = lo + 1;
    else pick = (lo & 1) ? lo + 1 : lo;
    return (uint8_t)(sign | pick);
  }
}

uint8_t o_fp8_encode_brute(float x, int fmt) {
  table_t t;
  build_table(fmt, &t);
  return brute_encode(&t, x);
}

typedef struct {
  int fmt; uint64_t b0, b1; uint64_t mismatches; uint32_t first_bad; int has_bad;
  const table_t* t;
} ex_job;

static void* ex_worker(void* p) {
  ex_job* j = (ex_job*)p;
  for (uint64_t b = j->b0; b < j->b1; ++b) {
    uint32_t u = (uint32_t)b;
    float x; memcpy(&x, &u, 4);
    if (o_fp8_encode(x, j->fmt) != brute_encode(j->t, x)) {
      if (!j->has_bad) { j->has_bad = 1; j->first_bad = u; }
      j->mismatches++;
    }
  }
  return NULL;
}

/* Compare the bit encoder against the brute-force encoder on every binary32
 * pattern in [lo, hi).  Returns the mismatch count; *first_bad gets the
 * first mismatching pattern (0xFFFFFFFF if none). */
uint64_t o_encode_exhaustive(int fmt, uint64_t lo, uint64_t hi, int nthreads,
                             uint32_t* first_bad) {
  table_t t;
  pthread_t th[256];
  ex_job jobs[256];
  uint64_t total = 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  build_table(fmt, &t);
  *first_bad = 0xFFFFFFFFu;
  for (int i = 0; i < nthreads; ++i) {
    jobs[i].fmt = fmt; jobs[i].t = &t; jobs[i].mismatches = 0; jobs[i].has_bad = 0;
    jobs[i].b0 = lo + (hi - lo) * (uint64_t)i / (uint64_t)nthreads;
    jobs[i].b1 = lo + (hi - lo) * (uint64_t)(i + 1) / (uint64_t)nthreads;
  }
  for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, ex_worker, &jobs[i]);
  ex_worker(&jobs[0]);
  for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
  for (int i = 0; i < nthreads; ++i) {
    total += jobs[i].mismatches;
    if (jobs[i].has_bad && *first_bad == 0xFFFFFFFFu) *first_bad = jobs[i].first_bad;
  }
  return total;
}
