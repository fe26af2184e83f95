// kvq_attn.h -- device helpers shared by the paged decode-attention kernels
// of libkvq.so (gfx950): cross-lane reductions, agent-scope partial-result
// accesses, the on-chip enumeration of split-K work items, and buffer
// descriptors for page chunks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// DPP lane moves inside a row of 16 lanes (VALU, no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kRowMirror = 0x140;  // lane i <-> 15-i within 16
template <int R>
constexpr int kRowRor = 0x120 + R;  // rotate right by R within 16

// Lane exchange across rows of 16 / halves of 32 (gfx950 permlane swaps,
// VALU only): with both operands equal, the pair returned holds the value of
// lane l and of lane l^16 (resp. l^32), so their sum is the 2-lane sum.
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum over aligned groups of W consecutive lanes (W a power of two <= 64):
// each step adds the partner that holds the sum of the neighbouring half.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (W >= 2) v += dpp<kQuadXor1>(v);
  if constexpr (W >= 4) v += dpp<kQuadXor2>(v);
  if constexpr (W >= 8) v += dpp<kHalfMirror>(v);
  if constexpr (W >= 16) v += dpp<kRowMirror>(v);
  if constexpr (W >= 32) v = sum_xor16(v);
  if constexpr (W >= 64) v = sum_xor32(v);
  return v;
}
// Sum / max over the lanes with equal (lane mod S): rotations by S, 2S, ...
// inside each row of 16 visit every such lane once, then across rows.
template <int S>
__device__ __forceinline__ float stride_sum(float v) {
  if constexpr (S <= 1) v += dpp<kRowRor<1>>(v);
  if constexpr (S <= 2) v += dpp<kRowRor<2>>(v);
  if constexpr (S <= 4) v += dpp<kRowRor<4>>(v);
  if constexpr (S <= 8) v += dpp<kRowRor<8>>(v);
  if constexpr (S <= 16) v = sum_xor16(v);
  if constexpr (S <= 32) v = sum_xor32(v);
  return v;
}
template <int S>
__device__ __forceinline__ float stride_max(float v) {
  if constexpr (S <= 1) v = fmaxf(v, dpp<kRowRor<1>>(v));
  if constexpr (S <= 2) v = fmaxf(v, dpp<kRowRor<2>>(v));
  if constexpr (S <= 4) v = fmaxf(v, dpp<kRowRor<4>>(v));
  if constexpr (S <= 8) v = fmaxf(v, dpp<kRowRor<8>>(v));
  if constexpr (S <= 16) v = max_xor16(v);
  if constexpr (S <= 32) v = max_xor32(v);
  return v;
}

// Split-K partials cross workgroups on different XCDs: agent-scope relaxed
// accesses keep them coherent without flushing the L2.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int clamped_len(const DecodeArgs& a, int b) {
  int L = a.seq_lens[b];
  const int64_t cap = (int64_t)a.max_pages * kPageSize;
  if (L < 0) L = 0;
  if ((int64_t)L > cap) L = (int)cap;
  return L;
}

// Exclusive scan of per-sequence item counts into s_prefix[0..B], by all 256
// threads: each sums a contiguous range of sequences, the ranges are scanned
// with wave shuffles and one LDS exchange, then written out.
// The same over the lengths len(b) (the slab's extend attention numbers its
// work by new token; see kvq_mla.hip).
template <int kThreads, typename LenFn>
__device__ void build_prefix_with(const DecodeArgs& a, int item_tokens, int units, int* s_prefix,
                                  int* s_wave, LenFn len) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = a.batch;
  const int per = (B + kThreads - 1) / kThreads;
  const int b0 = tid * per, b1 = min(b0 + per, B);
  int local = 0;
  for (int b = b0; b < b1; ++b) local += (len(b) + item_tokens - 1) / item_tokens * units;
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += s_wave[w];
  int run = base + incl - local;
  for (int b = b0; b < b1; ++b) {
    s_prefix[b] = run;
    run += (len(b) + item_tokens - 1) / item_tokens * units;
  }
  if (tid == kThreads - 1) s_prefix[B] = base + incl;
  __syncthreads();
}

template <int kThreads>
__device__ void build_prefix(const DecodeArgs& a, int item_tokens, int units, int* s_prefix,
                             int* s_wave) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = a.batch;
  const int per = (B + kThreads - 1) / kThreads;
  const int b0 = tid * per, b1 = min(b0 + per, B);
  int local = 0;
  for (int b = b0; b < b1; ++b) local += (clamped_len(a, b) + item_tokens - 1) / item_tokens * units;
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += s_wave[w];
  int run = base + incl - local;
  for (int b = b0; b < b1; ++b) {
    s_prefix[b] = run;
    run += (clamped_len(a, b) + item_tokens - 1) / item_tokens * units;
  }
  if (tid == kThreads - 1) s_prefix[B] = base + incl;
  __syncthreads();
}

// How the GQA kernels size their work items (see DecodePlan).
struct ItemRule {
  int step, min_pages, cap_pages, target;
};

// Tokens per work item under rule r for a batch holding `pages` pages in
// all, `units` items per chunk of a sequence.
__host__ __device__ inline int rule_item_tokens(const ItemRule& r, int64_t pages, int units) {
  const int64_t work = pages * units;
  int64_t ip = (work + r.target - 1) / r.target;
  ip = (ip + r.step - 1) / r.step * r.step;
  ip = ip < r.min_pages ? r.min_pages : (ip > r.cap_pages ? r.cap_pages : ip);
  return (int)ip * kPageSize;
}

// Pages per work item from the batch's actual lengths, the same in every
// workgroup: about r.target items over all (sequence, unit) pairs, a
// multiple of r.step, within [r.min_pages, r.cap_pages]; then the exclusive
// scan of per-sequence item counts into s_prefix.  Returns tokens per item.
template <int kThreads>
__device__ int plan_items(const DecodeArgs& a, const ItemRule& r, int units, int* s_prefix,
                          int* s_wave) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = a.batch;
  const int per = (B + kThreads - 1) / kThreads;
  const int b0 = tid * per, b1 = min(b0 + per, B);
  int pages = 0;
  for (int b = b0; b < b1; ++b) pages += (clamped_len(a, b) + kPageSize - 1) / kPageSize;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) pages += __shfl_xor(pages, off, 64);
  if (lane == 0) s_wave[wave] = pages;
  __syncthreads();
  int64_t total = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) total += s_wave[w];
  __syncthreads();  // s_wave is reused by the scan
  const int item_tokens = rule_item_tokens(r, total, units);
  build_prefix<kThreads>(a, item_tokens, units, s_prefix, s_wave);
  return item_tokens;
}

// Inclusive prefix sum over the 64 lanes: DPP shifts inside each row of 16
// (lanes shifted in from outside the row read 0), then the totals of the
// rows below are added from scalar reads of their last lanes.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// The work list of a batch of at most 64 sequences, built by one wave alone
// (every wave builds the same one; no LDS, no barrier): lane b < batch gets
// the number of items before sequence b, and *total the number of items.
// Same rule as plan_items.  `len` is clamped_len(a, lane) for lane < batch,
// else 0 (loaded by the caller, which may issue other loads after it).
__device__ __forceinline__ int plan_items_wave(const ItemRule& r, int units, int len, int* pfx,
                                               int* total) {
  const int pages = (len + kPageSize - 1) / kPageSize;
  const int all_pages = __builtin_amdgcn_readlane(wave_incl_scan(pages), 63);
  const int item_tokens = rule_item_tokens(r, all_pages, units);
  const int items = (len + item_tokens - 1) / item_tokens * units;
  const int incl = wave_incl_scan(items);
  *pfx = incl - items;
  *total = __builtin_amdgcn_readlane(incl, 63);
  return item_tokens;
}

// Sequence of work item `item` in a list built by plan_items_wave: the last
// b < batch with pfx(b) <= item (pfx is non-decreasing over the lanes).
__device__ __forceinline__ int wave_item_seq(int pfx, int batch, int item) {
  const uint64_t m = __builtin_amdgcn_ballot_w64((int)(threadIdx.x & 63) < batch && pfx <= item);
  return __builtin_popcountll(m) - 1;
}

// exp2(x - m) that is 0 (not NaN) when both are -inf.  The raw hardware
// exp2 is enough here: arguments are <= 0 and tiny results may flush to 0.
__device__ __forceinline__ float exp2_rel(float x, float m) {
  return (x == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(x - m);
}

// Query rows of a kv head.  Column c (0 .. n_hg * gt) of kv head kvh is,
// for the decode, query head kvh * G + c of sequence b; for extend attention
// it is new token i = c / G of the sequence, head kvh * G + c % G (rows are
// token-major, so a 16-column tile holds 16 / G consecutive new tokens).
// query_row gives its row of q / out ([rows][Hq]), -1 for a padding column;
// query_end the exclusive end of the positions it may attend to: the length
// L for the decode, P + i + 1 for new token i at position P + i = L - E + i.
__device__ __forceinline__ int64_t query_row(const DecodeArgs& a, int b, int kvh, int c, int G) {
  if (!a.q_start) return (int64_t)b * a.n_q_heads + kvh * G + c;
  const int qs = a.q_start[b], E = min(a.q_start[b + 1] - qs, a.max_new);
  const int i = c / G;
  return i < E ? (int64_t)(qs + i) * a.n_q_heads + kvh * G + (c - i * G) : -1;
}
__device__ __forceinline__ int query_end(const DecodeArgs& a, int b, int L, int c, int G) {
  if (!a.q_start) return L;
  const int E = a.q_start[b + 1] - a.q_start[b];
  const int i = c / G;
  return i < min(E, a.max_new) ? L - E + i + 1 : 0;
}

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer descriptor, gfx9 family
constexpr int kNonTemporal = 2;         // cache policy: streaming (read once)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRsrcWord3);
}

}  // namespace kvq
