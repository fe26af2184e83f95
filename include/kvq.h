/*
 * kvq.h -- C ABI of libkvq.so: a block-scaled 8-bit paged KV cache for
 * AMD Instinct MI355X (gfx950).
 *
 * K/V rows are stored as 8-bit codes (OCP fp8 e4m3fn, or int8 "q8_0") with one
 * IEEE fp16 scale per 32 consecutive elements along head_dim, 17/16 bytes per
 * element against 2 for bf16; the quantize-on-store kernel writes them, and
 * the paged decode-attention kernel reads them back through a page table,
 * dequantizing before the dot products because the scale varies along the
 * reduction dimension.
 *
 * Sources (web pages, cited by title and section):
 *   [PR103] "feat(kvcache): 8-bit KV cache (q8_0 / fp8_e4m3) behind
 *           --kv-cache-dtype" (FreeToken #103) and the review comment on it.
 *   [PR113] "feat(kvcache): 8-bit DSV4 window/compressed KV behind
 *           --kv-cache-dtype" (FreeToken #113).
 *   [PR126] "Add fp8 KV-cache quantization (--kv-dtype)" (FreeToken #126).
 *   [PR25]  "Experimental FP8 KV Cache" (llama.cpp fork #25).
 *
 * Conventions for every call:
 *   - Pointers marked "device" point to GPU memory the caller allocated and
 *     owns; the library never allocates, frees or synchronizes, and keeps no
 *     state between calls other than the thread-local error message (and
 *     kvq_paged_decode_noalloc's fixed device array).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and runs asynchronously; results are valid once the stream reaches it.
 *   - Arguments are validated on the host before anything is launched; a call
 *     that returns an error has enqueued nothing and written nothing.  The
 *     message is available from kvq_last_error() on the calling thread.
 *   - Values that live in device memory (slots, page ids, sequence lengths)
 *     cannot be checked without a synchronization; the kernels instead skip
 *     what is out of range, as documented per argument.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
/* A HIP stream (the same type as hipStream_t). */
typedef struct ihipStream_t* kvq_stream_t;

/* Storage type of a pool.  KVQ_BF16 stores rows unchanged (no scales); the
 * two block-scaled 8-bit types share one scale layout, store kernel and
 * dequant path [PR103 §What].  The two cast types store each element itself
 * as an 8-bit float (a per-tensor scale of 1.0) and have no scale buffer:
 * one byte per element, twice bf16's tokens in the same bytes [PR126 "Add fp8
 * KV-cache quantization (--kv-dtype)" §Summary (e4m3 or e5m2), §How it works
 * (the store casts with scale 1.0), §Benchmark (2.00x the token budget)].
 * The cast rounds to nearest even; a magnitude beyond the format's largest
 * finite value stores that value (448 for e4m3, 57344 for e5m2), the same
 * saturation the block-scaled store applies.  Inputs must be finite.
 * KVQ_FP8_DS_MLA is the 656-byte row of the 576-wide MLA latent [PR25
 * "Experimental FP8 KV Cache": a 656-byte fp8 row laid out as in vLLM; the
 * page gives no field list, and the one taken is]: bytes 0..511 the e4m3fn
 * codes of latent elements 0..511, bytes 512..527 four fp32 scales (scale j =
 * max|x| / 448 over elements 128j .. 128j+127, an fp32 division; each code the
 * RNE e4m3 of the clamped fp32 quotient x / scale; a zero tile stores scale 0
 * and zero codes), bytes 528..655 the 64 rope elements as bf16.  One row per
 * token (n_heads 1, head_dim 576), no scale buffer; the MLA slab decode
 * (kvq_paged_decode with k_pool == v_pool) and kvq_sparse_mla_decode read it. */
typedef enum {
  KVQ_BF16 = 0,          /* 2 bytes per element, no scale buffer                  */
  KVQ_FP8_E4M3 = 1,      /* e4m3fn codes, scale = max|x| / 448 per 32-block       */
  KVQ_Q8_0 = 2,          /* int8 codes in [-127, 127], scale = max|x| / 127       */
  KVQ_FP8_E4M3_CAST = 3, /* e4m3fn code of x itself, no scale buffer              */
  KVQ_FP8_E5M2_CAST = 4, /* e5m2 code of x itself, no scale buffer               */
  KVQ_FP8_DS_MLA = 5     /* 656-byte MLA row: 512 e4m3 + 4 fp32 scales + 64 bf16 */
} kvq_dtype;

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_ARG = -1,         /* a bad argument (null pointer, bad size, ...)       */
  KVQ_ERR_UNSUPPORTED = -2, /* a valid request this build does not implement      */
  KVQ_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required         */
  KVQ_ERR_HIP = -4          /* the HIP runtime reported an error at launch        */
} kvq_status;

/* Elements per scale block along head_dim [PR103 §What; PR113 §What this adds]. */
#define KVQ_BLOCK 32

/* ---------------------------------------------------------------------------
 * Pool layout (fixed; the pages give none):
 *   codes : [num_pages][n_heads][page_size][head_dim], 1 byte per element
 *           (2 bytes of bf16 for KVQ_BF16); each (page, head) chunk of
 *           page_size rows is contiguous.
 *   scales: [num_pages][n_heads][page_size][head_dim / 32] fp16 (IEEE binary16
 *           bit patterns), a separate buffer beside the codes [PR103 §What:
 *           parallel scale buffers; PR113 §What this adds: one scale array
 *           beside the single MLA slab].  The block-scaled types only; the
 *           cast types and KVQ_BF16 have none.
 * A token lives at slot = page * page_size + offset.  For the MLA latent slab
 * (one KV head, K and V the same row) n_heads = 1 and head_dim = 576.
 * KVQ_FP8_DS_MLA: [num_pages][1][page_size][656] bytes, each row as described
 * at kvq_dtype (codes, scales and rope together); no scale buffer.
 * ------------------------------------------------------------------------- */

/* Bytes of one pool (codes + scales) for one of K or V.  This is the cost
 * model: the caller should size allocations and token budgets with this same
 * function, so that the budget and the pool cannot disagree [PR113 §One
 * ordering trap worth knowing about; PR103 §What: unit_bytes()/kv_cost() on
 * effective bytes].  Host-only, pure.  *scale_bytes (nullable) receives the
 * bytes of the scale buffer (0 for KVQ_BF16, the cast types and the 656-byte
 * row); the code buffer is the return value minus that.
 * Returns -1 (and sets the error message) on invalid arguments:
 * num_pages < 0, page_size < 1, n_heads < 1, head_dim < 1, head_dim not a
 * multiple of 32 for an 8-bit type, or an unknown dtype. */
int64_t kvq_pool_bytes(kvq_dtype dtype, int64_t num_pages, int page_size, int n_heads,
                       int head_dim, int64_t* scale_bytes);

/* Quantize-on-store [PR103 §What: store kernel, per-block max-abs -> codes +
 * scales; review §"A bug on sm_89": clamp, then round to nearest even for
 * e4m3, half away from zero for q8_0; PR113 §What this adds].
 *
 * For every token n with a valid slot and every head h, each 32-element block
 * x of row src[n][h] is stored as
 *     s = fp16_rne(fp32(max|x| / M)), M = 448 (e4m3) or 127 (q8_0),
 *         held at 65504 if the quotient exceeds it;
 *     code_i = round(clamp(fp32(x_i / s), -M, M)), e4m3: nearest even,
 *         q8_0: half away from zero; s == 0 gives all-zero codes.
 * Both quotients are IEEE fp32 divisions; the result is bit-exact and
 * deterministic.  An infinite element makes max|x| / M infinite, so its
 * block's scale is held at 65504: the element stores +-M and the others
 * their quotient by 65504.  NaN elements are not supported (their codes and
 * their block's scale are unspecified).  KVQ_BF16 copies the row unchanged.  The cast types store
 *     code_i = round(clamp(x_i, -M, M)), nearest even, M = 448 (e4m3) or
 *         57344 (e5m2), and write no scale.
 *
 *   k_src, v_src : device, bf16 [n_tokens][..] rows; head h of token n starts
 *                  at element n * src_token_stride + h * head_dim.  v_src may
 *                  be NULL (then v_pool / v_scales are ignored): this stores
 *                  only K, e.g. the single MLA slab.  Both must be 16-byte
 *                  aligned and src_token_stride a multiple of 8 elements,
 *                  at least n_heads * head_dim.
 *   slot_mapping : device int32 [n_tokens]; slot < 0 or >= num_pages *
 *                  page_size is skipped.  Two tokens with the same slot in
 *                  one call leave that slot undefined.
 *   k_pool/v_pool, k_scales/v_scales : device, layout above; scales are
 *                  ignored (may be NULL) for KVQ_BF16 and the cast types.
 * Supported: head_dim a multiple of 32 (any multiple of 8 for KVQ_BF16) up
 * to 1024, n_heads >= 1, page_size 1..1024, n_tokens >= 0 (0 is a no-op).
 * Errors: KVQ_ERR_ARG, KVQ_ERR_HIP. */
int kvq_store(kvq_dtype dtype, const void* k_src, const void* v_src,
              int64_t src_token_stride, const int32_t* slot_mapping, int64_t n_tokens,
              int n_heads, int head_dim, int page_size, int64_t num_pages, void* k_pool,
              uint16_t* k_scales, void* v_pool, uint16_t* v_scales, kvq_stream_t stream);

/* Gather-dequantize rows to bf16 [PR103 §What: dequant path; PR126 §How it
 * works: dequantize on read].  out[n][h][d] = bf16_rne(code * s) for the row
 * at slot_mapping[n]; an invalid slot gives a row of zeros.  code * s is exact
 * in fp32, so the only rounding is the final one to bf16 (s = 1 for the cast
 * types, whose codes are exact in bf16).
 *   pool, scales : device, layout above (scales ignored for KVQ_BF16 and the
 *                  cast types).
 *   out_bf16     : device bf16 [n_tokens][n_heads][head_dim], 16-byte aligned.
 * Supported and errors as kvq_store. */
int kvq_dequant(kvq_dtype dtype, const void* pool, const uint16_t* scales,
                const int32_t* slot_mapping, int64_t n_tokens, int n_heads, int head_dim,
                int page_size, int64_t num_pages, void* out_bf16, kvq_stream_t stream);

/* Workspace bytes kvq_paged_decode needs for these shapes (split-K partial
 * results and arrival counters), for any storage type.  The shapes name the
 * kernel: n_kv_heads == 1 with head_dim_v == 512 is the shared 576/512 slab,
 * any other shape has head_dim_qk == head_dim_v.  0 if no storage type
 * supports the shapes (see kvq_paged_decode).  Host-only, pure. */
size_t kvq_paged_decode_workspace_bytes(int batch, int n_q_heads, int n_kv_heads,
                                        int head_dim_v, int max_pages, int page_size);

/* Paged decode attention: one bf16 query token per sequence against the
 * quantized pool [PR103 §What: dequant inside the attention kernels behind a
 * QUANT switch, K/V dequantized before the dot because the scale runs along
 * head_dim; PR113 §Testing: split-k decode kernel, masked (-1) columns].
 *
 * For sequence b and query head h, with kv head g = h / (n_q_heads /
 * n_kv_heads), the valid tokens are t < min(seq_lens[b], max_pages *
 * page_size) whose page id page_table[b][t / page_size] lies in
 * [0, num_pages); any other id (-1 in particular) removes that page.  With
 * k_t, v_t the dequantized rows of head g,
 *     z_t = sm_scale * q[b][h] . k_t,
 *     out[b][h] = sum_t softmax(z)_t v_t     (bf16),
 *     lse[b][h] = log sum_t exp(z_t)         (fp32, natural log).
 * No valid token: out = 0, lse = -inf.
 *
 *   q          : device bf16 [batch][n_q_heads][head_dim_qk], 16-byte aligned.
 *   k_pool/v_pool, k_scales/v_scales : device, layout above, head_dim =
 *                head_dim_qk for K and head_dim_v for V.  The shared MLA slab
 *                [PR113 §What this adds; PR25, the SPARSE_MLA_DECODE shape]:
 *                pass v_pool == k_pool and v_scales == k_scales with
 *                n_kv_heads = 1; V is then the first head_dim_v elements of
 *                each K row.
 *   page_table : device int32 [batch][pt_stride]; columns >= max_pages are
 *                never read.
 *   seq_lens   : device int32 [batch]; negative counts as 0.
 *   seq_lens_host : host int32 [batch] holding the same values, or NULL.
 *                The kernels plan the split from seq_lens on the device
 *                either way (the device values decide the result); given
 *                the host copy, the launch is sized to the exact number of
 *                work items instead of an upper bound.  Read before the
 *                call returns.
 *   out_bf16   : device bf16 [batch][n_q_heads][head_dim_v].
 *   lse        : device fp32 [batch][n_q_heads], or NULL.
 *   workspace  : device, at least kvq_paged_decode_workspace_bytes() bytes,
 *                256-byte aligned, zero-filled before its first use.  It
 *                holds split-K partial results and per-(sequence, kv head)
 *                arrival counters; every completed call leaves the counters
 *                at zero again, so a workspace is zeroed once, not per call.
 *                Calls that share a workspace must not overlap.
 * Supported: page_size 16; separate K/V with head_dim_qk == head_dim_v in
 * {32, 64, 128, 256} and any n_q_heads a multiple of n_kv_heads, batch
 * 1..4096; the shared slab with head_dim_qk 576, head_dim_v 512, n_kv_heads
 * 1, n_q_heads a multiple of 16 up to 128, batch 1..1024 and max_pages up to
 * 32768; max_pages >= 1; num_pages >= 1.  For the slab, K enters the dot
 * products as bf16(code * scale), as in the pages' dequantize-to-bf16 path.
 * Errors: KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE, KVQ_ERR_HIP. */
int kvq_paged_decode(kvq_dtype dtype, const void* q, const void* k_pool,
                     const uint16_t* k_scales, const void* v_pool, const uint16_t* v_scales,
                     const int32_t* page_table, int64_t pt_stride, const int32_t* seq_lens,
                     const int32_t* seq_lens_host, int batch, int n_q_heads, int n_kv_heads,
                     int head_dim_qk, int head_dim_v, int page_size, int max_pages,
                     int64_t num_pages, float sm_scale, void* out_bf16, float* lse,
                     void* workspace, size_t workspace_bytes, kvq_stream_t stream);

/* Decode with append: each sequence's new token is stored, then every
 * sequence is decoded, in one call -- the per-layer work of a decode step
 * [PR126 "Add fp8 KV-cache quantization (--kv-dtype)" §How it works (the
 * incoming bf16 k/v rows are converted to the pool type as they are written
 * to the cache; attention dequantizes on read); PR103 "feat(kvcache): 8-bit
 * KV cache (q8_0 / fp8_e4m3) behind --kv-cache-dtype" §What (the store
 * kernel quantizes, the attention kernels read the quantized pool)].
 *
 * The result, the pools and the lse are exactly those of
 *     kvq_store(dtype, new_k, new_v, new_token_stride, slot, batch,
 *               n_kv_heads, head_dim_qk, page_size, num_pages, k_pool,
 *               k_scales, v_pool, v_scales, stream);
 *     kvq_paged_decode(... the same pools, page table, lengths ...);
 * with slot[b] = page_table[b][(L - 1) / page_size] * page_size + (L - 1) %
 * page_size for L = seq_lens[b] (the new token is the last position of its
 * sequence, already counted in seq_lens), and slot[b] = -1 -- nothing stored
 * -- when L < 1, L > max_pages * page_size, or that page id lies outside
 * [0, num_pages).
 *
 *   new_k, new_v : device bf16 [batch][n_kv_heads][head_dim_qk] with
 *                  new_token_stride elements between sequences (>=
 *                  n_kv_heads * head_dim_qk, a multiple of 8), 16-byte
 *                  aligned.  For the shared MLA slab (k_pool == v_pool) new_v
 *                  is NULL and new_k holds the 576-wide rows; otherwise new_v
 *                  is required.
 *   k_pool, k_scales, v_pool, v_scales : as kvq_paged_decode, written.
 *   Every other argument: as kvq_paged_decode.
 * With separate K/V and fewer than 8 query heads per kv head the new rows are
 * quantized and stored inside the decode launch (by the work item that
 * attends that position, with the store kernel's arithmetic); the other
 * shapes enqueue the store kernel, then the decode.  Two sequences whose new
 * tokens share a slot race, as they would in kvq_store.
 * Errors: as kvq_paged_decode, and KVQ_ERR_ARG for a null new_k, a new_v
 * that does not match the pool sharing, or a bad stride or alignment. */
int kvq_paged_decode_append(kvq_dtype dtype, const void* q, const void* new_k,
                            const void* new_v, int64_t new_token_stride, void* k_pool,
                            uint16_t* k_scales, void* v_pool, uint16_t* v_scales,
                            const int32_t* page_table, int64_t pt_stride, const int32_t* seq_lens,
                            const int32_t* seq_lens_host, int batch, int n_q_heads,
                            int n_kv_heads, int head_dim_qk, int head_dim_v, int page_size,
                            int max_pages, int64_t num_pages, float sm_scale, void* out_bf16,
                            float* lse, void* workspace, size_t workspace_bytes,
                            kvq_stream_t stream);

/* kvq_paged_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The arguments and the result are kvq_paged_decode's, without
 * the workspace: the split-K partials and arrival counters live in the
 * library's own array of 64 MiB per device (a static device array, held by
 * every GPU the library runs on until the process ends; its address is taken
 * once per device on the first call there).  Each call first clears the
 * arrival counters its plan uses (a small fill kernel on `stream`), then
 * decodes.  Calls on one GPU share the array and leave their partials in
 * it, so calls that overlap on one GPU (other streams, other threads) race;
 * calls on different GPUs do not.  Shapes whose plan needs more than the
 * array holds (kvq_paged_decode_workspace_bytes() > 64 MiB: for the 576/512
 * slab with 128 heads and 10240 pages, a batch above 3; for 16 q / 8 kv heads
 * of head_dim 128 over 8192 pages, a batch above about 250) are refused with
 * KVQ_ERR_WORKSPACE before anything is enqueued.  Nothing is allocated.
 * Errors: as kvq_paged_decode. */
int kvq_paged_decode_noalloc(kvq_dtype dtype, const void* q, const void* k_pool,
                             const uint16_t* k_scales, const void* v_pool,
                             const uint16_t* v_scales, const int32_t* page_table,
                             int64_t pt_stride, const int32_t* seq_lens,
                             const int32_t* seq_lens_host, int batch, int n_q_heads,
                             int n_kv_heads, int head_dim_qk, int head_dim_v, int page_size,
                             int max_pages, int64_t num_pages, float sm_scale, void* out_bf16,
                             float* lse, kvq_stream_t stream);

/* Workspace bytes kvq_sparse_mla_decode needs: the split-K partials of the
 * slab decode over the lists (each list split into work items of up to 1024
 * entries).  0 if the shapes are invalid (see kvq_sparse_mla_decode).
 * Host-only. */
size_t kvq_sparse_mla_decode_workspace_bytes(kvq_dtype dtype, int batch, int n_q_heads,
                                             int topk);

/* Sparse top-k decode over the shared MLA slab [PR25 "Experimental FP8 KV
 * Cache": SPARSE_MLA_DECODE, D=576 Hq=128 Hkv=1 Dv=512, K=256 tokens selected
 * out of the cache for each query; PR113 "feat(kvcache): 8-bit DSV4
 * window/compressed KV behind --kv-cache-dtype" §What this adds (one slab, K
 * and V the same row), §Testing (masked (-1) columns)].
 *
 * Sequence b attends only to the tokens listed in topk_idx[b][0 .. topk):
 * token positions within the sequence, read through the page table as in
 * kvq_paged_decode.  An entry is taken when 0 <= t < seq_lens[b] (clamped to
 * max_pages * page_size) and its page id lies in [0, num_pages); any other
 * entry (-1 pads a short list) is skipped.  Taken entries count as listed (a
 * position listed twice counts twice).  With k_t the taken rows and v_t their
 * first 512 elements:
 *     z_t = sm_scale * q[b][h] . k_t,  out[b][h] = sum_t softmax(z)_t v_t,
 *     lse[b][h] = log sum_t exp(z_t);  no entry taken: out = 0, lse = -inf.
 *
 *   q         : device bf16 [batch][n_q_heads][576], 16-byte aligned.
 *   slab, scales : device, the pool layout above with n_heads = 1 and
 *               head_dim = 576 (scales ignored, may be NULL, for KVQ_BF16 and
 *               the cast types).
 *   topk_idx  : device int32 [batch][topk_stride], topk_stride >= topk.
 *   page_table, seq_lens, out_bf16 ([batch][n_q_heads][512]), lse: as
 *               kvq_paged_decode.
 *   workspace : device, >= kvq_sparse_mla_decode_workspace_bytes(), 256-byte
 *               aligned; overwritten by every call (no zeroing needed).
 * Supported: topk 1..2048, n_q_heads a multiple of 16 up to 128, batch up to
 * 1024, page_size 16.  The slab decode reads the listed rows in place (an
 * entry not taken is a masked token).  Errors: KVQ_ERR_ARG,
 * KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE, KVQ_ERR_HIP; validation completes
 * before any launch. */
int kvq_sparse_mla_decode(kvq_dtype dtype, const void* q, const void* slab,
                          const uint16_t* scales, const int32_t* page_table, int64_t pt_stride,
                          const int32_t* seq_lens, const int32_t* topk_idx, int64_t topk_stride,
                          int topk, int batch, int n_q_heads, int page_size, int max_pages,
                          int64_t num_pages, float sm_scale, void* out_bf16, float* lse,
                          void* workspace, size_t workspace_bytes, kvq_stream_t stream);

/* Workspace bytes kvq_extend_attention needs (the split-K partials and
 * counters of the matrix-core kernel over max_new_tokens x G query rows per
 * kv head).  When the batch's query-row tiles alone give every resident
 * workgroup several work items (long prefill: batch x n_kv_heads x tile
 * groups >= 2048), each tile group attends to its whole sequence in one work
 * item and the workspace holds no partials (a few KB).  0 if the shapes are
 * invalid (see kvq_extend_attention).  Host-only. */
size_t kvq_extend_attention_workspace_bytes(kvq_dtype dtype, int batch, int n_q_heads,
                                            int n_kv_heads, int head_dim, int page_size,
                                            int max_pages, int max_new_tokens);

/* Causal extend (prefill) attention over the quantized pool [PR103
 * "feat(kvcache): 8-bit KV cache (q8_0 / fp8_e4m3) behind --kv-cache-dtype"
 * §What: the quantized pool feeds the prefill / extend attention kernels as
 * well as the decode; PR113 "feat(kvcache): 8-bit DSV4 window/compressed KV
 * behind --kv-cache-dtype" §Testing: prefill, masked (-1) columns].
 *
 * The new tokens' K and V are already in the pool (kvq_store).  Sequence b
 * holds L = seq_lens[b] tokens (clamped to max_pages * page_size), of which
 * the last E = q_start[b+1] - q_start[b] are new; new token i sits at position
 * P + i, P = L - E, and attends to positions 0 .. P + i of its sequence:
 *     z_t = sm_scale * q[j][h] . k_t[kv(h)],  out[j][h] = sum_t softmax(z)_t v_t,
 *     lse[j][h] = log sum_t exp(z_t),  j = q_start[b] + i, kv(h) = h / (Hq/Hkv);
 * a token with no visible position (P + i < 0, or all pages masked): out = 0,
 * lse = -inf.  Masked (-1) page-table entries are skipped as in the decode.
 * E = L (no prefix) is a prefill.
 *
 *   q          : device bf16 [T][n_q_heads][head_dim], T = q_start[batch],
 *                16-byte aligned: the new tokens of every sequence, back to back.
 *   q_start    : device int32 [batch + 1]: q_start[0] = 0, nondecreasing, each
 *                difference at most max_new_tokens (rows past max_new_tokens of
 *                a sequence are not written).
 *   k_pool, v_pool, scales, page_table, seq_lens, num_pages: as kvq_paged_decode:
 *                separate K and V pools with head_dim 64, 128 or 256, or the
 *                shared 576/512 slab (k_pool == v_pool, k_scales == v_scales,
 *                n_kv_heads 1, head_dim 576; batch x max_new_tokens at most
 *                1024), whose V is the first 512 elements of each row.
 *   out_bf16   : device bf16 [T][n_q_heads][head_dim] (the slab: [T][n_q_heads]
 *                [512]); lse: device fp32 [T][n_q_heads] or NULL.
 *   workspace  : as kvq_paged_decode, sized by
 *                kvq_extend_attention_workspace_bytes(): zeroed once, left at
 *                zero by every call; calls sharing it must not overlap.  It
 *                holds split-K partials for every tile and grows linearly with
 *                max_new_tokens (8 sequences x 1024 pages, 16/8 heads, head_dim
 *                128: 21 MB at 64 new tokens, 1.4 GB at 4096).
 * Over the slab each new token runs as one query of the slab decode (its 128
 * or fewer heads are one matrix-core tile set), over its own causal length.
 * With separate pools the query rows of a kv head (token-major, max_new_tokens
 * x G of them) run on
 * the matrix cores in tiles of 16, two tiles per work item up to head_dim 128;
 * each work item streams the K/V of its token range once for its tiles.
 * Errors: KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE, KVQ_ERR_HIP;
 * validation completes before any launch. */
int kvq_extend_attention(kvq_dtype dtype, const void* q, const int32_t* q_start,
                         int max_new_tokens, const void* k_pool, const uint16_t* k_scales,
                         const void* v_pool, const uint16_t* v_scales, const int32_t* page_table,
                         int64_t pt_stride, const int32_t* seq_lens, int batch, int n_q_heads,
                         int n_kv_heads, int head_dim, int page_size, int max_pages,
                         int64_t num_pages, float sm_scale, void* out_bf16, float* lse,
                         void* workspace, size_t workspace_bytes, kvq_stream_t stream);

/* Message for the last non-OK return on the calling thread ("" if none). */
const char* kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
