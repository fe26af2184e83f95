// kvq_internal.h -- declarations shared by the host entry points (kvq_api.cpp)
// and the HIP kernel files of libkvq.so.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// QT_DSM: the 656-byte MLA row (512 e4m3 codes, four fp32 scales one per 128
// latent elements, 64 bf16 rope elements), one per token, no scale buffer.
enum { QT_BF16 = 0, QT_FP8 = 1, QT_Q8 = 2, QT_FP8C = 3, QT_BF8C = 4, QT_DSM = 5 };
constexpr int kDsmRow = 656, kDsmLatent = 512, kDsmTile = 128;
// block-scaled 8-bit codes (a scale buffer beside the pool)
__host__ __device__ constexpr bool qt_scaled(int qt) { return qt == QT_FP8 || qt == QT_Q8; }
// 8-bit float codes (e4m3 or e5m2), block-scaled or cast
__host__ __device__ constexpr bool qt_f8(int qt) {
  return qt == QT_FP8 || qt == QT_FP8C || qt == QT_BF8C;
}

// Token rows per page supported by the decode kernels.
constexpr int kPageSize = 16;
// Largest batch the decode kernels index through their on-chip work list.
constexpr int kMaxBatch = 4096;
// Waves per workgroup of the GQA decode kernel.
constexpr int kDecodeWaves = 4;
// Compute units the split planner assumes (MI355X); the plan must not depend
// on the device so that the workspace query and the call agree.
constexpr int kPlanCUs = 256;
// A work item spans at most 64 pages per wave (256 for 4 waves).
constexpr int kMaxItemPages = 256;
// The last workgroup of a (sequence, kv head, head group) merges the chunk
// partials itself when they hold at most this many bytes; otherwise a
// separate merge kernel runs.
constexpr int kFusedMergeMaxBytes = 64 * 1024;
// Extend attention takes one work item per (sequence, kv head, tile group)
// over the whole sequence when there are at least kWholeUnitsPerWorkgroup
// such units per resident workgroup (every workgroup then has several items
// and nothing needs splitting) and the split plan's partials would exceed
// kWholeMinPartialBytes.
constexpr int kWholeUnitsPerWorkgroup = 4;
constexpr int64_t kWholeMinPartialBytes = (int64_t)1 << 30;
// Chunk weights the merge keeps in LDS: chunks * heads per item.
constexpr int kMergeMaxWeights = 4096;

// Shared MLA latent slab: row width (K), V width (leading part of the row),
// tokens per LDS tile, and the planner's limits (batch held in LDS beside
// the tiles, pages per work item, chunks the merge weighs per sequence).
constexpr int kMlaDqk = 576;
constexpr int kMlaDv = 512;
constexpr int kMlaTile = 32;
constexpr int kMlaMaxBatch = 1024;
constexpr int kMlaMaxItemPages = 64;
constexpr int kMlaMaxChunks = 512;

// GQA decode geometry shared by the planner and the kernels: bytes of one
// (page, kv head) of codes and of scales, and how many pages a wave streams
// through its LDS buffer per step (about 8.5 KB of K and V per step).
__host__ __device__ constexpr int gqa_elem_bytes(int qtype) { return qtype == QT_BF16 ? 2 : 1; }
__host__ __device__ constexpr int gqa_code_bytes(int qtype, int d) {
  return kPageSize * d * gqa_elem_bytes(qtype);
}
__host__ __device__ constexpr int gqa_scale_bytes(int qtype, int d) {
  return qt_scaled(qtype) ? kPageSize * (d / 32) * 2 : 0;
}
constexpr int kGqaStepBytes = 8704;  // K and V bytes a wave loads per step (at least a page)
constexpr int kGqaDepth = 2;         // steps in flight per wave, including the one computed
__host__ __device__ constexpr int gqa_pages_per_step(int qtype, int d) {
  return (kGqaStepBytes / (2 * (gqa_code_bytes(qtype, d) + gqa_scale_bytes(qtype, d)))) < 1
             ? 1
             : kGqaStepBytes / (2 * (gqa_code_bytes(qtype, d) + gqa_scale_bytes(qtype, d)));
}

struct StoreArgs {
  int qtype;
  const uint16_t* src[2];  // K, V (V may be null)
  int64_t stride;          // elements between tokens
  const int32_t* slots;
  int64_t n_tokens;
  int n_heads, head_dim, page_size;
  int64_t num_pages;
  uint8_t* pool[2];
  uint16_t* scales[2];
  // Append mode (seq_lens set, slots unused): token b is the new token of
  // sequence b, stored at position seq_lens[b] - 1 through the page table;
  // nothing is stored for a length of 0 or past max_pages pages, or for a
  // masked page.
  const int32_t* seq_lens = nullptr;
  const int32_t* page_table = nullptr;
  int64_t pt_stride = 0;
  int max_pages = 0;
};

struct DequantArgs {
  int qtype;
  const uint8_t* pool;
  const uint16_t* scales;
  const int32_t* slots;
  int64_t n_tokens;
  int n_heads, head_dim, page_size;
  int64_t num_pages;
  uint16_t* out;
};

hipError_t launch_store(const StoreArgs& a, hipStream_t s);
hipError_t launch_dequant(const DequantArgs& a, hipStream_t s);
// Test export: e4m3 codes of the fp32 bit patterns first .. first + count - 1.
hipError_t launch_debug_e4m3(uint32_t first, int64_t count, uint8_t* out, hipStream_t s);

// ---- paged decode --------------------------------------------------------------

enum DecodeKind { DK_GQA = 0, DK_MLA = 1 };

struct DecodePlan {
  int kind;
  int gt;             // query heads (columns) per tile
  int tn = 1;         // tiles per work item (extend attention: 2 when they fill)
  int n_hg;           // head groups per kv head (G / gt)
  int item_pages;     // pages per split-K work item (the MLA slab; GQA: the smallest)
  // GQA: the kernels size work items from the actual lengths, about `target`
  // items over the batch: ceil(pages x units / target), rounded up to a
  // multiple of `step`, within [min_pages, cap_pages]
  int step, min_pages, cap_pages, target;
  bool fused_merge;   // merge inside the split kernel (else a merge kernel)
  bool mfma;          // GQA: wide query groups on the matrix-core kernel
  bool whole;         // extend: one item per (sequence, unit) over the whole
                      // sequence (no split-K partials in the workspace)
  int64_t max_items;  // upper bound on work items (sizes the workspace)
  size_t off_prefix, off_count, off_ml, off_acc, bytes;  // workspace layout
};

struct DecodeArgs {
  int qtype;
  const uint16_t* q;
  const uint8_t* k_pool;
  const uint16_t* k_scales;
  const uint8_t* v_pool;
  const uint16_t* v_scales;
  const int32_t* page_table;
  int64_t pt_stride;
  const int32_t* seq_lens;
  int batch, n_q_heads, n_kv_heads, head_dim_qk, head_dim_v, max_pages;
  int64_t num_pages;
  float sm_scale;
  uint16_t* out;
  float* lse;
  void* workspace;
  // Extend attention (null for the decode): the new tokens' query rows of
  // sequence b are q_start[b] .. q_start[b+1]-1 of q and out ([rows][Hq][D]),
  // at most max_new of them per sequence.
  const int32_t* q_start = nullptr;
  int max_new = 0;
  // Decode with append (kvq_paged_decode_append): the bf16 K and V rows of
  // each sequence's new token, new_kv[t] + b * new_stride ([n_kv_heads][D]),
  // are quantized and written to position seq_lens[b] - 1 (as the append
  // store above) before that position is attended; the pools are then
  // written, so the pool pointers above are the caller's writable ones.
  const uint16_t* new_kv[2] = {nullptr, nullptr};
  int64_t new_stride = 0;
  // Host-side only: the exact number of work items when the caller passed
  // the lengths on the host too (0: unknown); the launch then holds no
  // workgroup beyond it.  The kernels themselves plan from seq_lens.
  int64_t items_hint = 0;
  // Sparse decode over the slab (null otherwise): sequence b attends to the
  // positions listed at topk[b * topk_stride + i], i < topk_k, instead of
  // its first seq_lens[b] positions.
  const int32_t* topk = nullptr;
  int64_t topk_stride = 0;
  int topk_k = 0;
};

constexpr int kExtendMaxNew = 65536;  // new tokens per sequence, extend attention

// Host-only planning: returns false (with a message) for unsupported shapes.
// ext_new > 0 plans extend attention with at most ext_new new tokens per
// sequence (the matrix-core kernel, ext_new x G query rows per kv head).
bool plan_decode(int qtype, int batch, int n_q_heads, int n_kv_heads, int head_dim_qk,
                 int head_dim_v, int page_size, int max_pages, DecodePlan* plan,
                 const char** why, int ext_new = 0);

// The VALU decode kernels of one storage type; kvq_decode.hip is compiled
// once per type (-DKVQ_DECODE_QT), each object defining its own.
template <int QT>
hipError_t launch_gqa_decode_typed(const DecodeArgs& a, const DecodePlan& p, int num_cus,
                                   hipStream_t s);
template <>
hipError_t launch_gqa_decode_typed<QT_BF16>(const DecodeArgs&, const DecodePlan&, int, hipStream_t);
template <>
hipError_t launch_gqa_decode_typed<QT_FP8>(const DecodeArgs&, const DecodePlan&, int, hipStream_t);
template <>
hipError_t launch_gqa_decode_typed<QT_Q8>(const DecodeArgs&, const DecodePlan&, int, hipStream_t);
template <>
hipError_t launch_gqa_decode_typed<QT_FP8C>(const DecodeArgs&, const DecodePlan&, int, hipStream_t);
template <>
hipError_t launch_gqa_decode_typed<QT_BF8C>(const DecodeArgs&, const DecodePlan&, int, hipStream_t);
inline hipError_t launch_gqa_decode(const DecodeArgs& a, const DecodePlan& p, int num_cus,
                                    hipStream_t s) {
  switch (a.qtype) {
    case QT_BF16: return launch_gqa_decode_typed<QT_BF16>(a, p, num_cus, s);
    case QT_FP8: return launch_gqa_decode_typed<QT_FP8>(a, p, num_cus, s);
    case QT_FP8C: return launch_gqa_decode_typed<QT_FP8C>(a, p, num_cus, s);
    case QT_BF8C: return launch_gqa_decode_typed<QT_BF8C>(a, p, num_cus, s);
    default: return launch_gqa_decode_typed<QT_Q8>(a, p, num_cus, s);
  }
}
// The separate split-K merge of the GQA kernels (plan.fused_merge == false).
hipError_t launch_gqa_merge(const DecodeArgs& a, const DecodePlan& p, hipStream_t s);
hipError_t launch_gqa_mfma_decode(const DecodeArgs& a, const DecodePlan& p, int num_cus,
                                  hipStream_t s);
hipError_t launch_mla_decode(const DecodeArgs& a, const DecodePlan& p, int num_cus,
                             hipStream_t s);

// ---- the library's own scratch array (kvq_noalloc.hip) ------------------------
// Size of the per-device array that kvq_paged_decode_noalloc uses as its
// workspace, its device address on the current device (taken once per device
// with hipGetSymbolAddress), and a fill kernel that zeroes `words` 32-bit
// words at p.
size_t scratch_bytes();
hipError_t scratch_pointer(void** p);
hipError_t launch_zero_words(void* p, size_t words, hipStream_t s);

// ---- sparse top-k decode over the MLA slab -------------------------------------
// The listed rows of every sequence are gathered into a compact slab in the
// workspace (kk rows per sequence: k rounded up to a page), which the slab
// decode then attends to in full.
constexpr int kSparseMaxK = 2048;

// The sparse decode: the slab kernel's plan over lists of k entries (k
// rounded up to a page), which is also the whole workspace.
struct SparseLayout {
  int kk;
  DecodePlan dense;
  size_t bytes;
};

bool plan_sparse(int qtype, int batch, int n_q_heads, int k, SparseLayout* lay, const char** why);

}  // namespace kvq
