/*
 * kvq_oracle.c -- plain, slow CPU oracle for the block-scaled 8-bit paged KV
 * cache (quantize-on-store, dequantize, paged decode attention).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call this file:
 * only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg load
 * it.  It shares no code, header, table or constant with the HIP library.
 *
 * Sources (web pages, cited by title and section):
 *   [PR103]  "feat(kvcache): 8-bit KV cache (q8_0 / fp8_e4m3) behind
 *            --kv-cache-dtype" (FreeToken pull request #103), and the
 *            review comment on it ("A bug on sm_89: the fp8 store does not
 *            round to nearest", "End-to-end numbers").
 *   [PR113]  "feat(kvcache): 8-bit DSV4 window/compressed KV behind
 *            --kv-cache-dtype" (FreeToken pull request #113).
 *   [PR126]  "Add fp8 KV-cache quantization (--kv-dtype)" (FreeToken #126).
 *   [PR25]   "Experimental FP8 KV Cache" (llama.cpp fork pull request #25).
 *
 * Precision: the pages fix the storage formats (e4m3 / int8 codes, an IEEE
 * binary16 scale per 32 elements) but not the arithmetic of the quotient.
 * The reading taken: the block max-abs is divided by the format maximum in
 * IEEE fp32, rounded once more to fp16; each element is divided by that fp16
 * scale in IEEE fp32 and the quotient is rounded onto the code grid.  Attention
 * is computed in double over exactly dequantized K/V.
 *
 * Every rounding here goes through one definition, round_to_grid(), which is
 * IEEE round-to-nearest-even onto a binary floating-point grid with p
 * fraction bits and minimum normal exponent emin, done with exact double
 * arithmetic and rint().  Build without -ffast-math and with
 * -ffp-contract=off so that every float operation rounds as written.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KVO_BF16 0
#define KVO_FP8_E4M3 1
#define KVO_Q8_0 2
/* Per-tensor scale 1.0: each element cast to fp8 itself, no scale buffer
 * [PR126 §How it works: the store casts the bf16 k/v to the pool's fp8 dtype
 * with scale 1.0; §Summary: fp8_e4m3 or fp8_e5m2]. */
#define KVO_FP8_E4M3_CAST 3
#define KVO_FP8_E5M2_CAST 4
/* The 656-byte MLA row [PR25 "Experimental FP8 KV Cache": a 656-byte fp8 row
 * for the 576-wide latent, laid out as in vLLM].  The page does not give the
 * fields; the reading taken: bytes 0..511 the e4m3fn codes of latent elements
 * 0..511, bytes 512..527 four fp32 scales (scale j for elements 128j ..
 * 128j+127, amax/448 rounded once to fp32), bytes 528..655 the 64 rope
 * elements as bf16, unquantized.  One such row per token (n_heads = 1,
 * head_dim = 576), no scale buffer. */
#define KVO_FP8_DS_MLA 5
#define KVO_DS_ROW 656
#define KVO_DS_LATENT 512
#define KVO_DS_TILE 128

/* Quantization block length along head_dim, and the two format maxima:
 * 448 is the largest finite e4m3 magnitude, 127 the int8 limit [PR103 §What;
 * PR113 §What this adds]. */
#define KVO_BLOCK 32
#define KVO_E4M3_MAX 448.0f
#define KVO_Q8_MAX 127.0f
#define KVO_F16_MAX 65504.0
/* Largest finite e5m2 magnitude: 1.75 * 2^15 (the exponent field 31 holds
 * the infinities and NaNs). */
#define KVO_E5M2_MAX 57344.0f

/* ------------------------------------------------------------------------ */
/* Rounding onto a binary floating-point grid.                               */
/* ------------------------------------------------------------------------ */

/* Round a >= 0 to the nearest value of a binary format with p fraction bits
 * and minimum normal exponent emin (no upper limit is applied here), ties to
 * the value whose last fraction bit is 0.  Below 2^emin the grid spacing is
 * fixed at 2^(emin-p) (subnormals).  a / quantum is exact in double because
 * the quantum is a power of two; rint() rounds half to even. */
static double round_to_grid(double a, int p, int emin) {
  if (a == 0.0) return 0.0;
  int e;
  frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
  e -= 1;       /* a = g * 2^e, g in [1, 2)   */
  if (e < emin) e = emin;
  double quantum = ldexp(1.0, e - p);
  return rint(a / quantum) * quantum;
}

/* ---- IEEE binary16 ------------------------------------------------------ */

/* fp16 bits -> value (exact). */
double kvo_f16_value(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp(1.0 + m / 1024.0, e - 15);
  return s ? -v : v;
}

/* value -> fp16 bits, round to nearest even, overflow to infinity. */
uint16_t kvo_f16_from_double(double x) {
  uint16_t s = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (isnan(x)) return 0x7e00;
  double r = round_to_grid(a, 10, -14);
  if (r >= 65536.0) return s | 0x7c00; /* rounds past the largest finite */
  if (r < ldexp(1.0, -14)) return s | (uint16_t)(r * 16777216.0); /* m*2^-24 */
  int e;
  double f = frexp(r, &e); /* r = f*2^e, f in [0.5,1) */
  int E = e - 1 + 15;
  uint16_t m = (uint16_t)((f * 2.0 - 1.0) * 1024.0);
  return s | (uint16_t)(E << 10) | m;
}

/* ---- bfloat16 (8-bit exponent, 7 fraction bits) -------------------------- */

double kvo_bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* finite value -> bf16 bits, round to nearest even. */
uint16_t kvo_bf16_from_double(double x) {
  uint16_t s = signbit(x) ? 0x8000 : 0;
  if (isnan(x)) return 0x7fc0;
  double r = round_to_grid(fabs(x), 7, -126);
  if (r >= ldexp(1.0, 128)) return s | 0x7f80;
  if (r < ldexp(1.0, -126)) return s | (uint16_t)(r * ldexp(1.0, 133));
  int e;
  double f = frexp(r, &e);
  int E = e - 1 + 127;
  uint16_t m = (uint16_t)((f * 2.0 - 1.0) * 128.0);
  return s | (uint16_t)(E << 7) | m;
}

/* ---- OCP fp8 e4m3fn ------------------------------------------------------
 * Bias 7, 3 fraction bits, no infinities, 0x7F/0xFF are NaN, so the largest
 * finite magnitude is 0x7E = 1.75*2^8 = 448 [PR103 §What: s = max/448].
 * Normal codes: (1 + m/8) * 2^(e-7), e = 1..15; subnormal: m * 2^-9. */
double kvo_e4m3_value(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 0xf, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* Encode v (|v| <= 448, finite) as the nearest e4m3fn code, ties to the code
 * with an even last fraction bit (round-to-nearest-even, the rounding the
 * review comment on [PR103] says a correct store must do, §"A bug on sm_89").
 * The sign is kept, so a negative value that rounds to zero encodes as 0x80. */
uint8_t kvo_e4m3_encode(float v) {
  uint8_t s = signbit(v) ? 0x80 : 0;
  double r = round_to_grid(fabs((double)v), 3, -6);
  if (r < ldexp(1.0, -6)) return s | (uint8_t)(r * 512.0); /* m * 2^-9 */
  int e;
  double f = frexp(r, &e);
  int E = e - 1 + 7;
  uint8_t m = (uint8_t)((f * 2.0 - 1.0) * 8.0);
  return s | (uint8_t)(E << 3) | m;
}

/* ---- fp8 e5m2 ------------------------------------------------------------
 * Bias 15, 2 fraction bits, IEEE-like: exponent field 31 is infinity (m = 0)
 * or NaN.  Normal codes: (1 + m/4) * 2^(e-15), e = 1..30; subnormal: m * 2^-16.
 * [PR126 §Summary: --kv-dtype fp8_e5m2.] */
double kvo_e5m2_value(uint8_t c) {
  int s = c >> 7, e = (c >> 2) & 0x1f, m = c & 3;
  double v;
  if (e == 31) v = m ? NAN : INFINITY;
  else if (e == 0)
    v = ldexp((double)m, -16);
  else
    v = ldexp(1.0 + m / 4.0, e - 15);
  return s ? -v : v;
}

/* Encode v (|v| <= 57344, finite) as the nearest e5m2 code, ties to the code
 * with an even last fraction bit; the sign is kept (-0 encodes as 0x80). */
uint8_t kvo_e5m2_encode(float v) {
  uint8_t s = signbit(v) ? 0x80 : 0;
  double r = round_to_grid(fabs((double)v), 2, -14);
  if (r < ldexp(1.0, -14)) return s | (uint8_t)(r * 65536.0); /* m * 2^-16 */
  int e;
  double f = frexp(r, &e);
  int E = e - 1 + 15;
  uint8_t m = (uint8_t)((f * 2.0 - 1.0) * 4.0);
  return s | (uint8_t)(E << 2) | m;
}

/* The cast store of one element (per-tensor scale 1.0).  The pages leave a
 * value beyond the format's range open (their k/v "sit well inside" it); the
 * reading taken is the saturation the block-scaled store applies: clamp to
 * the largest finite magnitude, then round to nearest even. */
uint8_t kvo_cast_encode(int qtype, float x) {
  float M = (qtype == KVO_FP8_E5M2_CAST) ? KVO_E5M2_MAX : KVO_E4M3_MAX;
  if (x > M) x = M;
  if (x < -M) x = -M;
  return (qtype == KVO_FP8_E5M2_CAST) ? kvo_e5m2_encode(x) : kvo_e4m3_encode(x);
}

/* ---- q8_0 ----------------------------------------------------------------
 * Round half away from zero (the GGUF Q8_0 convention the review comment on
 * [PR103] names, §"A bug on sm_89"), for |v| <= 127.  |v| + 0.5 is exact in
 * double, so floor() gives the exact half-away result. */
int8_t kvo_q8_encode(float v) {
  double a = floor(fabs((double)v) + 0.5);
  return (int8_t)(signbit(v) ? -a : a);
}

/* ---- block scale -----------------------------------------------------------
 * s = max-abs / 448 (e4m3) or / 127 (q8_0), held as IEEE fp16 [PR103 §What;
 * PR113 §What this adds].  Reading: fp32 division, then fp16 round-to-nearest-
 * even; a quotient beyond the largest finite fp16 is held at 65504 so that
 * the block saturates rather than becoming infinite.  Returns fp16 bits. */
uint16_t kvo_block_scale(int qtype, float amax) {
  float M = (qtype == KVO_Q8_0) ? KVO_Q8_MAX : KVO_E4M3_MAX;
  float q = amax / M; /* IEEE fp32 division */
  if ((double)q > KVO_F16_MAX) return 0x7bff;
  return kvo_f16_from_double((double)q);
}

/* Quantize one block of n (= 32) bf16 values: the per-block max-abs gives the
 * scale, each element is divided by the stored scale in fp32, clamped to the
 * format maximum and rounded onto the code grid [PR103 §What and review
 * §"A bug on sm_89" (clamp, then round)].  A zero scale (all-zero block, or a
 * max-abs too small for fp16) stores all-zero codes. */
void kvo_quantize_block(int qtype, const uint16_t* x, int n, uint8_t* codes,
                        uint16_t* scale_out) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) {
    float a = fabsf((float)kvo_bf16_value(x[i]));
    if (a > amax) amax = a;
  }
  uint16_t sh = kvo_block_scale(qtype, amax);
  *scale_out = sh;
  float s = (float)kvo_f16_value(sh);
  for (int i = 0; i < n; ++i) {
    if (s == 0.0f) {
      codes[i] = 0;
      continue;
    }
    float xi = (float)kvo_bf16_value(x[i]);
    float v = xi / s; /* IEEE fp32 division by the stored scale */
    if (qtype == KVO_Q8_0) {
      if (v > KVO_Q8_MAX) v = KVO_Q8_MAX;
      if (v < -KVO_Q8_MAX) v = -KVO_Q8_MAX;
      codes[i] = (uint8_t)kvo_q8_encode(v);
    } else {
      if (v > KVO_E4M3_MAX) v = KVO_E4M3_MAX;
      if (v < -KVO_E4M3_MAX) v = -KVO_E4M3_MAX;
      codes[i] = kvo_e4m3_encode(v);
    }
  }
}

/* Exact value of one stored element: decoded code times the fp16 scale.
 * Both factors have few significant bits, so the product is exact in double
 * (and in fp32).  bf16 pools store the value itself. */
double kvo_element_value(int qtype, uint8_t code, uint16_t scale) {
  if (qtype == KVO_FP8_E4M3_CAST) return kvo_e4m3_value(code);
  if (qtype == KVO_FP8_E5M2_CAST) return kvo_e5m2_value(code);
  if (qtype == KVO_Q8_0) return (double)(int8_t)code * kvo_f16_value(scale);
  return kvo_e4m3_value(code) * kvo_f16_value(scale);
}

/* ------------------------------------------------------------------------ */
/* A plain parallel-for over independent work units.                        */
/* ------------------------------------------------------------------------ */

typedef void (*kvo_unit_fn)(void* ctx, int64_t unit);
typedef struct {
  kvo_unit_fn fn;
  void* ctx;
  int64_t begin, end;
} kvo_range;

static void* kvo_run_range(void* p) {
  kvo_range* r = (kvo_range*)p;
  for (int64_t u = r->begin; u < r->end; ++u) r->fn(r->ctx, u);
  return NULL;
}

static void kvo_parallel_for(int64_t n, int threads, kvo_unit_fn fn, void* ctx) {
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  if (threads == 1 || n < 2) {
    for (int64_t u = 0; u < n; ++u) fn(ctx, u);
    return;
  }
  pthread_t tid[256];
  kvo_range rg[256];
  int64_t per = (n + threads - 1) / threads;
  int used = 0;
  for (int t = 0; t < threads; ++t) {
    int64_t b = t * per, e = b + per < n ? b + per : n;
    if (b >= e) break;
    rg[t].fn = fn;
    rg[t].ctx = ctx;
    rg[t].begin = b;
    rg[t].end = e;
    if (pthread_create(&tid[t], NULL, kvo_run_range, &rg[t]) != 0) {
      kvo_run_range(&rg[t]); /* run inline if a thread cannot be made */
      tid[t] = 0;
    }
    used = t + 1;
  }
  for (int t = 0; t < used; ++t)
    if (tid[t]) pthread_join(tid[t], NULL);
}

/* ------------------------------------------------------------------------ */
/* Store: quantize rows of new tokens into the paged pool.                   */
/* ------------------------------------------------------------------------ */
/* Pool layout: codes [num_pages][n_heads][page_size][head_dim] (1 byte per
 * element; 2 bytes of bf16 for KVO_BF16), scales [num_pages][n_heads]
 * [page_size][head_dim/32] fp16 beside it [PR103 §What: parallel scale
 * buffers; PR113 §What this adds: a single scale array beside the slab].
 * A slot is page*page_size + offset; slot < 0 or >= capacity is skipped. */

typedef struct {
  int qtype;
  const uint16_t* src;
  int64_t token_stride;
  const int32_t* slots;
  int n_heads, head_dim, page_size;
  int64_t num_pages;
  uint8_t* pool;
  uint16_t* scales;
} kvo_store_ctx;

static void kvo_store_unit(void* p, int64_t n) {
  kvo_store_ctx* c = (kvo_store_ctx*)p;
  int64_t slot = c->slots[n];
  if (slot < 0 || slot >= c->num_pages * (int64_t)c->page_size) return;
  int64_t page = slot / c->page_size, off = slot % c->page_size;
  int nb = c->head_dim / KVO_BLOCK;
  for (int h = 0; h < c->n_heads; ++h) {
    const uint16_t* row = c->src + n * c->token_stride + (int64_t)h * c->head_dim;
    int64_t r = (page * c->n_heads + h) * c->page_size + off; /* row index */
    if (c->qtype == KVO_BF16) {
      memcpy(c->pool + r * c->head_dim * 2, row, (size_t)c->head_dim * 2);
      continue;
    }
    if (c->qtype == KVO_FP8_E4M3_CAST || c->qtype == KVO_FP8_E5M2_CAST) {
      for (int d = 0; d < c->head_dim; ++d)
        c->pool[r * c->head_dim + d] = kvo_cast_encode(c->qtype, (float)kvo_bf16_value(row[d]));
      continue;
    }
    if (c->qtype == KVO_FP8_DS_MLA) {
      /* per 128-element tile of the latent: s = amax / 448 in fp32, each
       * element's fp32 quotient x / s clamped and rounded to nearest even on
       * the e4m3fn grid; a zero tile stores s = 0 and zero codes; the rope
       * part is copied */
      uint8_t* rp = c->pool + r * KVO_DS_ROW;
      for (int j = 0; j < KVO_DS_LATENT / KVO_DS_TILE; ++j) {
        float amax = 0.0f;
        for (int e = 0; e < KVO_DS_TILE; ++e) {
          float a = fabsf((float)kvo_bf16_value(row[j * KVO_DS_TILE + e]));
          if (a > amax) amax = a;
        }
        float sc = amax / KVO_E4M3_MAX;
        for (int e = 0; e < KVO_DS_TILE; ++e) {
          float x = (float)kvo_bf16_value(row[j * KVO_DS_TILE + e]);
          rp[j * KVO_DS_TILE + e] = (sc > 0.0f) ? kvo_e4m3_encode(x / sc) : 0;
        }
        memcpy(rp + KVO_DS_LATENT + 4 * j, &sc, 4);
      }
      memcpy(rp + KVO_DS_LATENT + 16, row + KVO_DS_LATENT, (size_t)(c->head_dim - KVO_DS_LATENT) * 2);
      continue;
    }
    for (int j = 0; j < nb; ++j)
      kvo_quantize_block(c->qtype, row + j * KVO_BLOCK, KVO_BLOCK,
                         c->pool + r * c->head_dim + j * KVO_BLOCK, c->scales + r * nb + j);
  }
}

void kvo_store(int qtype, const uint16_t* src, int64_t token_stride, const int32_t* slots,
               int64_t n_tokens, int n_heads, int head_dim, int page_size, int64_t num_pages,
               uint8_t* pool, uint16_t* scales, int threads) {
  kvo_store_ctx c = {qtype, src, token_stride, slots, n_heads, head_dim, page_size,
                     num_pages, pool, scales};
  kvo_parallel_for(n_tokens, threads, kvo_store_unit, &c);
}

/* ------------------------------------------------------------------------ */
/* Dequantize rows gathered by slot: exact value, returned as double, or      */
/* rounded once to bf16.  An invalid slot yields zeros.                       */
/* ------------------------------------------------------------------------ */

typedef struct {
  int qtype;
  const uint8_t* pool;
  const uint16_t* scales;
  const int32_t* slots;
  int n_heads, head_dim, page_size;
  int64_t num_pages;
  double* out_f64;
  uint16_t* out_bf16;
} kvo_deq_ctx;

static double kvo_pool_value(int qtype, const uint8_t* pool, const uint16_t* scales,
                             int64_t row, int head_dim, int d) {
  if (qtype == KVO_BF16) {
    uint16_t b;
    memcpy(&b, pool + (row * head_dim + d) * 2, 2);
    return kvo_bf16_value(b);
  }
  if (qtype == KVO_FP8_E4M3_CAST || qtype == KVO_FP8_E5M2_CAST)
    return kvo_element_value(qtype, pool[row * head_dim + d], 0);
  if (qtype == KVO_FP8_DS_MLA) { /* code x its tile's fp32 scale; the rope as stored */
    const uint8_t* rp = pool + row * KVO_DS_ROW;
    if (d >= KVO_DS_LATENT) {
      uint16_t b;
      memcpy(&b, rp + KVO_DS_LATENT + 16 + 2 * (d - KVO_DS_LATENT), 2);
      return kvo_bf16_value(b);
    }
    float sc;
    memcpy(&sc, rp + KVO_DS_LATENT + 4 * (d / KVO_DS_TILE), 4);
    return kvo_e4m3_value(rp[d]) * (double)sc;
  }
  int nb = head_dim / KVO_BLOCK;
  return kvo_element_value(qtype, pool[row * head_dim + d], scales[row * nb + d / KVO_BLOCK]);
}

static void kvo_deq_unit(void* p, int64_t n) {
  kvo_deq_ctx* c = (kvo_deq_ctx*)p;
  int64_t slot = c->slots[n];
  int valid = slot >= 0 && slot < c->num_pages * (int64_t)c->page_size;
  int64_t page = valid ? slot / c->page_size : 0, off = valid ? slot % c->page_size : 0;
  for (int h = 0; h < c->n_heads; ++h) {
    int64_t r = (page * c->n_heads + h) * c->page_size + off;
    for (int d = 0; d < c->head_dim; ++d) {
      double v = valid ? kvo_pool_value(c->qtype, c->pool, c->scales, r, c->head_dim, d) : 0.0;
      int64_t o = (n * c->n_heads + h) * (int64_t)c->head_dim + d;
      if (c->out_f64) c->out_f64[o] = v;
      if (c->out_bf16) c->out_bf16[o] = kvo_bf16_from_double(v);
    }
  }
}

void kvo_dequant(int qtype, const uint8_t* pool, const uint16_t* scales, const int32_t* slots,
                 int64_t n_tokens, int n_heads, int head_dim, int page_size, int64_t num_pages,
                 double* out_f64, uint16_t* out_bf16, int threads) {
  kvo_deq_ctx c = {qtype, pool, scales, slots, n_heads, head_dim, page_size, num_pages,
                   out_f64, out_bf16};
  kvo_parallel_for(n_tokens, threads, kvo_deq_unit, &c);
}

/* ------------------------------------------------------------------------ */
/* Paged decode attention, one query token per sequence.                      */
/* ------------------------------------------------------------------------ */
/* For sequence b and query head h (kv head g = h / (Hq/Hkv)): the valid tokens
 * are t < seq_len[b] whose page-table entry is a page id in [0, num_pages);
 * a -1 (or any out-of-range) entry removes the whole page [PR113 §Testing:
 * masked (-1) columns].  K and V rows are dequantized exactly (the scale runs
 * along head_dim, the reduction dimension, so the values are formed before
 * the dot product [PR103 §What]); z_t = sm_scale * q . k_t;
 * o = sum_t softmax(z)_t v_t; lse = log sum_t exp(z_t).  For the shared MLA
 * slab (v_pool == k_pool) V is the first head_dim_v elements of the same row
 * [PR113 §What this adds; PR25, the SPARSE_MLA_DECODE shape D=576, Dv=512].
 * No valid token: o = 0, lse = -inf.  Everything in double. */

typedef struct {
  int qtype;
  const uint16_t* q;
  const uint8_t *k_pool, *v_pool;
  const uint16_t *k_scales, *v_scales;
  const int32_t* page_table;
  int64_t pt_stride;
  const int32_t* seq_lens;
  int batch, n_q_heads, n_kv_heads, head_dim_qk, head_dim_v, page_size, max_pages;
  int64_t num_pages;
  double sm_scale;
  const int32_t* rows;
  double* out;
  double* lse;
} kvo_dec_ctx;

/* Attention of one query row over the first L positions of sequence b, for
 * query head h: scores, softmax and the weighted sum of V, as stated above. */
static void kvo_attend(const kvo_dec_ctx* c, int b, int h, int64_t L, const uint16_t* qrow,
                       double* o, double* lse_out) {
  int g = h / (c->n_q_heads / c->n_kv_heads);
  int shared = (c->v_pool == c->k_pool);
  int v_row_dim = shared ? c->head_dim_qk : c->head_dim_v;
  if (L < 0) L = 0;
  double* z = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
  char* ok = (char*)malloc((size_t)(L > 0 ? L : 1));
  double zmax = -INFINITY;
  /* pass 1: scores */
  for (int64_t t = 0; t < L; ++t) {
    int64_t page = c->page_table[(int64_t)b * c->pt_stride + t / c->page_size];
    ok[t] = page >= 0 && page < c->num_pages;
    if (!ok[t]) continue;
    int64_t r = (page * c->n_kv_heads + g) * c->page_size + t % c->page_size;
    double dot = 0.0;
    for (int d = 0; d < c->head_dim_qk; ++d)
      dot += kvo_bf16_value(qrow[d]) *
             kvo_pool_value(c->qtype, c->k_pool, c->k_scales, r, c->head_dim_qk, d);
    z[t] = c->sm_scale * dot;
    if (z[t] > zmax) zmax = z[t];
  }
  for (int d = 0; d < c->head_dim_v; ++d) o[d] = 0.0;
  if (zmax == -INFINITY) { /* no valid token */
    if (lse_out) *lse_out = -INFINITY;
    free(z);
    free(ok);
    return;
  }
  /* pass 2: weights and the weighted sum of V */
  double denom = 0.0;
  for (int64_t t = 0; t < L; ++t) {
    if (!ok[t]) continue;
    int64_t page = c->page_table[(int64_t)b * c->pt_stride + t / c->page_size];
    int64_t r = (page * c->n_kv_heads + g) * c->page_size + t % c->page_size;
    double w = exp(z[t] - zmax);
    denom += w;
    for (int d = 0; d < c->head_dim_v; ++d)
      o[d] += w * kvo_pool_value(c->qtype, c->v_pool, c->v_scales, r, v_row_dim, d);
  }
  for (int d = 0; d < c->head_dim_v; ++d) o[d] /= denom;
  if (lse_out) *lse_out = zmax + log(denom);
  free(z);
  free(ok);
}

static int64_t kvo_clamped_len(const kvo_dec_ctx* c, int b) {
  int64_t L = c->seq_lens[b];
  int64_t cap = (int64_t)c->max_pages * c->page_size;
  if (L > cap) L = cap;
  if (L < 0) L = 0;
  return L;
}

static void kvo_dec_unit(void* p, int64_t i) {
  kvo_dec_ctx* c = (kvo_dec_ctx*)p;
  int64_t row = c->rows ? c->rows[i] : i; /* row = b * Hq + h */
  int b = (int)(row / c->n_q_heads), h = (int)(row % c->n_q_heads);
  kvo_attend(c, b, h, kvo_clamped_len(c, b), c->q + row * (int64_t)c->head_dim_qk,
             c->out + i * (int64_t)c->head_dim_v, c->lse ? c->lse + i : NULL);
}

/* rows: optional list of (b * n_q_heads + h) to compute (NULL = all rows, in
 * order); out: double [n_rows][head_dim_v]; lse: double [n_rows] or NULL. */
void kvo_paged_decode(int qtype, const uint16_t* q, const uint8_t* k_pool,
                      const uint16_t* k_scales, const uint8_t* v_pool, const uint16_t* v_scales,
                      const int32_t* page_table, int64_t pt_stride, const int32_t* seq_lens,
                      int batch, int n_q_heads, int n_kv_heads, int head_dim_qk, int head_dim_v,
                      int page_size, int max_pages, int64_t num_pages, double sm_scale,
                      const int32_t* rows, int64_t n_rows, double* out, double* lse, int threads) {
  kvo_dec_ctx c = {qtype,      q,          k_pool,     v_pool,     k_scales,  v_scales,
                   page_table, pt_stride,  seq_lens,   batch,      n_q_heads, n_kv_heads,
                   head_dim_qk, head_dim_v, page_size, max_pages,  num_pages, sm_scale,
                   rows,       out,        lse};
  if (!rows) n_rows = (int64_t)batch * n_q_heads;
  kvo_parallel_for(n_rows, threads, kvo_dec_unit, &c);
}

/* ------------------------------------------------------------------------ */
/* Extend (prefill) attention over the quantized pool.                        */
/* ------------------------------------------------------------------------ */
/* The pool is read by prefill / extend attention as well as by the decode
 * [PR103 §What: the quantized path covers the four attention kernels;
 * PR113 §Testing: prefill].  Sequence b holds L_b = seq_lens[b] tokens in the
 * pool (clamped as in the decode), of which the last E_b = q_start[b+1] -
 * q_start[b] are new; their queries are rows q_start[b] .. q_start[b+1] - 1
 * of q ([rows][n_q_heads][head_dim]).  New token i sits at position
 * P_b + i, P_b = L_b - E_b, and attends causally to positions 0 .. P_b + i:
 * the decode of that query over the sequence's first P_b + i + 1 positions
 * (none when that is <= 0: o = 0, lse = -inf).  q_start[0] = 0, q_start is
 * nondecreasing; out and lse have q_start[batch] * n_q_heads rows. */

typedef struct {
  kvo_dec_ctx d;
  const int32_t* q_start;
} kvo_ext_ctx;

static void kvo_ext_unit(void* p, int64_t r) {
  kvo_ext_ctx* e = (kvo_ext_ctx*)p;
  const kvo_dec_ctx* c = &e->d;
  int64_t j = r / c->n_q_heads; /* query token */
  int h = (int)(r % c->n_q_heads);
  int b = 0;
  while (b + 1 < c->batch && e->q_start[b + 1] <= j) ++b;
  int64_t E = e->q_start[b + 1] - e->q_start[b];
  int64_t i = j - e->q_start[b];
  int64_t len = kvo_clamped_len(c, b) - E + i + 1;
  kvo_attend(c, b, h, len, c->q + r * (int64_t)c->head_dim_qk, c->out + r * (int64_t)c->head_dim_v,
             c->lse ? c->lse + r : NULL);
}

/* head_dim_v < head_dim with v_pool == k_pool: the shared MLA slab (V the
 * first head_dim_v elements of each row), as in the decode. */
void kvo_extend_attention(int qtype, const uint16_t* q, const int32_t* q_start,
                          const uint8_t* k_pool, const uint16_t* k_scales, const uint8_t* v_pool,
                          const uint16_t* v_scales, const int32_t* page_table, int64_t pt_stride,
                          const int32_t* seq_lens, int batch, int n_q_heads, int n_kv_heads,
                          int head_dim, int head_dim_v, int page_size, int max_pages,
                          int64_t num_pages, double sm_scale, double* out, double* lse,
                          int threads) {
  kvo_ext_ctx e;
  kvo_dec_ctx c = {qtype,     q,          k_pool,    v_pool,     k_scales,  v_scales,
                   page_table, pt_stride, seq_lens,  batch,      n_q_heads, n_kv_heads,
                   head_dim,  head_dim_v, page_size, max_pages,  num_pages, sm_scale,
                   NULL,      out,        lse};
  e.d = c;
  e.q_start = q_start;
  kvo_parallel_for((int64_t)q_start[batch] * n_q_heads, threads, kvo_ext_unit, &e);
}

/* ------------------------------------------------------------------------ */
/* Sparse top-k decode over the shared MLA slab.                              */
/* ------------------------------------------------------------------------ */
/* Sequence b attends only to the tokens listed in topk[b][0..k): positions
 * within the sequence, read through the page table [PR25 "Experimental FP8
 * KV Cache": SPARSE_MLA_DECODE D=576 Hq=128 Hkv=1 Dv=512 K=256].  An entry is
 * taken when 0 <= t < seq_len (clamped to max_pages * page_size) and its page
 * id is in [0, num_pages); other entries (-1 pads a list) are skipped [PR113
 * §Testing: masked (-1) columns].  Taken entries count as listed (a position
 * listed twice counts twice).  K is the whole row, V its first head_dim_v
 * elements; scores, softmax and the weighted sum in double, as above. */

typedef struct {
  int qtype;
  const uint16_t* q;
  const uint8_t* slab;
  const uint16_t* scales;
  const int32_t* page_table;
  int64_t pt_stride;
  const int32_t* seq_lens;
  const int32_t* topk;
  int64_t topk_stride;
  int k, n_q_heads, head_dim_qk, head_dim_v, page_size, max_pages;
  int64_t num_pages;
  double sm_scale;
  double* out;
  double* lse;
} kvo_sparse_ctx;

static void kvo_sparse_unit(void* p, int64_t row) {
  kvo_sparse_ctx* c = (kvo_sparse_ctx*)p;
  int b = (int)(row / c->n_q_heads);
  int64_t L = c->seq_lens[b];
  int64_t cap = (int64_t)c->max_pages * c->page_size;
  if (L > cap) L = cap;
  if (L < 0) L = 0;
  const uint16_t* qrow = c->q + row * (int64_t)c->head_dim_qk;
  int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(c->k > 0 ? c->k : 1));
  double* z = (double*)malloc(sizeof(double) * (size_t)(c->k > 0 ? c->k : 1));
  int n = 0;
  double zmax = -INFINITY;
  for (int i = 0; i < c->k; ++i) {
    int64_t t = c->topk[(int64_t)b * c->topk_stride + i];
    if (t < 0 || t >= L) continue;
    int64_t page = c->page_table[(int64_t)b * c->pt_stride + t / c->page_size];
    if (page < 0 || page >= c->num_pages) continue;
    int64_t r = page * c->page_size + t % c->page_size; /* one kv head */
    double dot = 0.0;
    for (int d = 0; d < c->head_dim_qk; ++d)
      dot += kvo_bf16_value(qrow[d]) *
             kvo_pool_value(c->qtype, c->slab, c->scales, r, c->head_dim_qk, d);
    rows[n] = r;
    z[n] = c->sm_scale * dot;
    if (z[n] > zmax) zmax = z[n];
    ++n;
  }
  double* o = c->out + row * (int64_t)c->head_dim_v;
  for (int d = 0; d < c->head_dim_v; ++d) o[d] = 0.0;
  if (n == 0) {
    if (c->lse) c->lse[row] = -INFINITY;
    free(rows);
    free(z);
    return;
  }
  double denom = 0.0;
  for (int j = 0; j < n; ++j) {
    double w = exp(z[j] - zmax);
    denom += w;
    for (int d = 0; d < c->head_dim_v; ++d)
      o[d] += w * kvo_pool_value(c->qtype, c->slab, c->scales, rows[j], c->head_dim_qk, d);
  }
  for (int d = 0; d < c->head_dim_v; ++d) o[d] /= denom;
  if (c->lse) c->lse[row] = zmax + log(denom);
  free(rows);
  free(z);
}

/* out: double [batch * n_q_heads][head_dim_v]; lse: double [batch * n_q_heads] or NULL. */
void kvo_sparse_mla_decode(int qtype, const uint16_t* q, const uint8_t* slab,
                           const uint16_t* scales, const int32_t* page_table, int64_t pt_stride,
                           const int32_t* seq_lens, const int32_t* topk, int64_t topk_stride,
                           int k, int batch, int n_q_heads, int head_dim_qk, int head_dim_v,
                           int page_size, int max_pages, int64_t num_pages, double sm_scale,
                           double* out, double* lse, int threads) {
  kvo_sparse_ctx c = {qtype,      q,           slab,      scales,    page_table, pt_stride,
                      seq_lens,   topk,        topk_stride, k,       n_q_heads,  head_dim_qk,
                      head_dim_v, page_size,   max_pages, num_pages, sm_scale,   out,
                      lse};
  kvo_parallel_for((int64_t)batch * n_q_heads, threads, kvo_sparse_unit, &c);
}

/* ------------------------------------------------------------------------ */
/* Bulk helpers for tests: apply the scalar encoders to arrays.               */
/* ------------------------------------------------------------------------ */

void kvo_e4m3_encode_array(const float* v, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = kvo_e4m3_encode(v[i]);
}
/* The fp32 values with bit patterns first, first + 1, ..., first + n - 1. */
void kvo_e4m3_encode_bits(uint32_t first, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t b = first + (uint32_t)i;
    float v;
    memcpy(&v, &b, sizeof v);
    out[i] = kvo_e4m3_encode(v);
  }
}
void kvo_q8_encode_array(const float* v, int64_t n, int8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = kvo_q8_encode(v[i]);
}
void kvo_cast_encode_array(int qtype, const float* v, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = kvo_cast_encode(qtype, v[i]);
}
