/*
 * kvq_debug.h -- test exports of libkvq.so.  Not needed to use the library:
 * they expose internals that the test suite checks against the CPU oracle.
 * Same conventions as kvq.h (validation before any launch, negative kvq_status
 * codes with a message from kvq_last_error()).
 */
#ifndef KVQ_DEBUG_H
#define KVQ_DEBUG_H

#include "kvq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The device's fp32 -> e4m3fn encoder, the one every stored e4m3 code goes
 * through (clamp to +-448, then round to nearest even by the gfx950 packed
 * conversion), applied to the fp32 values whose bit patterns are first_bits,
 * first_bits + 1, ..., first_bits + count - 1.  The conversion is the part of
 * the store that differs per GPU architecture [PR103 "feat(kvcache): 8-bit KV
 * cache (q8_0 / fp8_e4m3) behind --kv-cache-dtype", review §"A bug on sm_89":
 * the fp8 store did not round to nearest on one architecture], so the tests
 * run it over every fp32 in [-448, 448] against the oracle's encoder.
 *   out_codes : device uint8 [count], 4-byte aligned; code i at byte i.
 * count must be a multiple of 4 with first_bits + count <= 2^32.
 * Errors: KVQ_ERR_ARG, KVQ_ERR_HIP. */
int kvq_debug_e4m3_encode_range(uint32_t first_bits, int64_t count, uint8_t* out_codes,
                                kvq_stream_t stream);

/* The decode planner's choice for these shapes (host-only, pure): writes up
 * to n_out of, in order, kind (0 separate K/V, 1 the 576/512 slab), query
 * columns per tile, tiles per work item, head groups per kv head, pages per
 * item step, fewest pages per item, most pages per item, target item count,
 * upper bound on items, workspace bytes, pages per item (the slab), merge
 * inside the decode kernel (0/1), matrix-core kernel (0/1), extend items
 * over whole sequences with no split-K partials (0/1).  max_new_tokens
 * > 0 plans kvq_extend_attention over separate pools.  Returns the number of
 * values written, or KVQ_ERR_UNSUPPORTED for shapes the planner refuses. */
int kvq_debug_decode_plan(kvq_dtype dtype, int batch, int n_q_heads, int n_kv_heads,
                          int head_dim_qk, int head_dim_v, int max_pages, int max_new_tokens,
                          int64_t* out, int n_out);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_DEBUG_H */
