/*
 * sweep.c -- exhaustive checks of the oracle's scalar encoders, written
 * independently of the oracle (test-side code; the oracle never sees it).
 *
 * e4m3: the non-negative finite e4m3fn values are listed from their closed
 * form (k * 2^-9 for k < 8, then (1 + m/8) * 2^(e-7)), in code order, which is
 * also value order.  Every fp32 bit pattern from +0 up to 448 is visited in
 * increasing order while a cursor tracks the grid interval [G_i, G_i+1]
 * holding it; the expected code is the nearer end, and on an exact midpoint
 * the end whose code has a zero last bit.  Midpoints of e4m3 neighbours have
 * at most 5 significant bits, so comparing against them in fp32 is exact.
 *
 * q8_0: for every fp32 v in [0, 127] the expected code is the integer part,
 * plus one when the (exact) fractional part is at least one half.
 *
 * Negative inputs are checked through the sign bit: the code of -v must be
 * the code of v with its sign bit (e4m3) or sign (q8_0) flipped.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

typedef uint8_t (*e4m3_fn)(float);
typedef int8_t (*q8_fn)(float);

static float f_of(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static float grid[127];
static void build_grid(void) {
  int n = 0;
  for (int k = 0; k < 8; ++k) grid[n++] = ldexpf((float)k, -9);
  for (int e = 1; e <= 15; ++e)
    for (int m = 0; m < 8; ++m) {
      if (e == 15 && m == 7) break; /* NaN code */
      grid[n++] = ldexpf(1.0f + m / 8.0f, e - 7);
    }
}

typedef struct {
  uint32_t lo, hi; /* bit range [lo, hi] of non-negative floats */
  e4m3_fn e4;
  q8_fn q8;
  int64_t bad;
  uint32_t first_bad;
} job;

static void* e4m3_job(void* p) {
  job* j = (job*)p;
  int i = 0;
  float x0 = f_of(j->lo);
  while (i < 125 && grid[i + 1] <= x0) ++i;
  for (uint64_t u = j->lo; u <= j->hi; ++u) {
    float x = f_of((uint32_t)u);
    while (i < 125 && grid[i + 1] <= x) ++i;
    int exp_code;
    if (x == grid[i]) {
      exp_code = i;
    } else {
      float mid = (grid[i] + grid[i + 1]) * 0.5f; /* exact */
      if (x < mid)
        exp_code = i;
      else if (x > mid)
        exp_code = i + 1;
      else
        exp_code = (i % 2 == 0) ? i : i + 1;
    }
    int got = j->e4(x);
    int got_neg = j->e4(-x);
    if (got != exp_code || got_neg != (exp_code | 0x80)) {
      if (j->bad == 0) j->first_bad = (uint32_t)u;
      j->bad++;
    }
  }
  return NULL;
}

static void* q8_job(void* p) {
  job* j = (job*)p;
  for (uint64_t u = j->lo; u <= j->hi; ++u) {
    float x = f_of((uint32_t)u);
    int n = (int)x;             /* truncation, x < 128 */
    float frac = x - (float)n;  /* exact */
    int exp_code = frac >= 0.5f ? n + 1 : n;
    int got = j->q8(x);
    int got_neg = j->q8(-x);
    if (got != exp_code || got_neg != -exp_code) {
      if (j->bad == 0) j->first_bad = (uint32_t)u;
      j->bad++;
    }
  }
  return NULL;
}

static int64_t run(void* (*fn)(void*), uint32_t hi, e4m3_fn e4, q8_fn q8, int threads,
                   uint32_t* first_bad) {
  if (threads < 1) threads = 1;
  if (threads > 64) threads = 64;
  pthread_t t[64];
  job jb[64];
  uint64_t n = (uint64_t)hi + 1, per = (n + threads - 1) / threads;
  int used = 0;
  for (int k = 0; k < threads; ++k) {
    uint64_t lo = k * per;
    if (lo > hi) break;
    uint64_t h = lo + per - 1 > hi ? hi : lo + per - 1;
    jb[k] = (job){(uint32_t)lo, (uint32_t)h, e4, q8, 0, 0};
    pthread_create(&t[k], NULL, fn, &jb[k]);
    used = k + 1;
  }
  int64_t bad = 0;
  *first_bad = 0xffffffffu;
  for (int k = 0; k < used; ++k) {
    pthread_join(t[k], NULL);
    if (jb[k].bad && *first_bad == 0xffffffffu) *first_bad = jb[k].first_bad;
    bad += jb[k].bad;
  }
  return bad;
}

/* Mismatch count over every fp32 in [-448, 448]; *first_bad = first bad bits. */
int64_t sweep_e4m3(e4m3_fn enc, int threads, uint32_t* first_bad) {
  build_grid();
  uint32_t hi;
  float m = 448.0f;
  memcpy(&hi, &m, 4);
  return run(e4m3_job, hi, enc, 0, threads, first_bad);
}

/* Mismatch count over every fp32 in [-127, 127]. */
int64_t sweep_q8(q8_fn enc, int threads, uint32_t* first_bad) {
  uint32_t hi;
  float m = 127.0f;
  memcpy(&hi, &m, 4);
  return run(q8_job, hi, 0, enc, threads, first_bad);
}

/* The grid as built here, for the Python side's closed-form checks. */
void sweep_grid(float* out127) {
  build_grid();
  memcpy(out127, grid, sizeof grid);
}
