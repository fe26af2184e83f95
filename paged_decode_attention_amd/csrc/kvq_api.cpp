// kvq_api.cpp -- host entry points of libkvq.so: argument validation, split
// planning, workspace layout and kernel launches.  Everything here runs on
// the host; validation finishes before any HIP call, so a rejected call
// touches neither the device nor the stream.
//
// Sources: [PR113] "feat(kvcache): 8-bit DSV4 window/compressed KV behind
// --kv-cache-dtype" §Gating (reject up front with a clear message: head_dim a
// multiple of the 32-element block) and §One ordering trap worth knowing
// about (the cost model must agree with the pool); [PR103] "feat(kvcache):
// 8-bit KV cache (q8_0 / fp8_e4m3) behind --kv-cache-dtype" §What (effective
// bytes per element, gating) and its review comment §Gating; [PR126] "Add fp8
// KV-cache quantization (--kv-dtype)" §Scope / limitations (refuse unsupported
// requests with a clear error rather than corrupt the cache).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "kvq.h"
#include "kvq_debug.h"
#include "kvq_attn.h"
#include "kvq_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return KVQ_OK;
}

bool known_dtype(int d) {
  return d == KVQ_BF16 || d == KVQ_FP8_E4M3 || d == KVQ_Q8_0 || d == KVQ_FP8_E4M3_CAST ||
         d == KVQ_FP8_E5M2_CAST || d == KVQ_FP8_DS_MLA;
}
// the 656-byte MLA row: one head of 576 elements per token
bool dsm_shape_ok(int n_heads, int head_dim) { return n_heads == 1 && head_dim == kvq::kMlaDqk; }
// a scale buffer beside the pool (the block-scaled types)
bool scaled(int d) { return d == KVQ_FP8_E4M3 || d == KVQ_Q8_0; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int hip_fail(hipError_t e, const char* what) {
  return fail(KVQ_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

int num_cus_current() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Work items of a decode call from host copies of the lengths, by the rule
// the kernels apply to the device copies (at least 1, so that one workgroup
// still writes the outputs of empty sequences).
int64_t host_items(const kvq::DecodePlan& p, const kvq::DecodeArgs& a, const int32_t* lens) {
  const int64_t cap = (int64_t)a.max_pages * kvq::kPageSize;
  auto clamp_len = [&](int b) {
    int64_t L = lens[b];
    return L < 0 ? (int64_t)0 : (L > cap ? cap : L);
  };
  int64_t item_tokens, units = 1;
  if (p.kind == kvq::DK_MLA) {
    item_tokens = (int64_t)p.item_pages * kvq::kPageSize;
  } else {
    units = (int64_t)a.n_kv_heads * p.n_hg;
    int64_t pages = 0;
    for (int b = 0; b < a.batch; ++b) pages += (clamp_len(b) + kvq::kPageSize - 1) / kvq::kPageSize;
    item_tokens = kvq::rule_item_tokens(
        kvq::ItemRule{p.step, p.min_pages, p.cap_pages, p.target}, pages, (int)units);
  }
  int64_t items = 0;
  for (int b = 0; b < a.batch; ++b) items += (clamp_len(b) + item_tokens - 1) / item_tokens * units;
  return items < 1 ? 1 : items;
}

// Shared by kvq_store and kvq_dequant.
int check_rows(int dtype, int64_t n_tokens, int n_heads, int head_dim, int page_size,
               int64_t num_pages, const char* fn) {
  if (!known_dtype(dtype)) return fail(KVQ_ERR_ARG, "%s: unknown dtype %d", fn, dtype);
  if (n_tokens < 0) return fail(KVQ_ERR_ARG, "%s: n_tokens %lld < 0", fn, (long long)n_tokens);
  if (n_heads < 1) return fail(KVQ_ERR_ARG, "%s: n_heads %d < 1", fn, n_heads);
  if (head_dim < 1 || head_dim > 1024)
    return fail(KVQ_ERR_ARG, "%s: head_dim %d outside 1..1024", fn, head_dim);
  if (dtype != KVQ_BF16 && head_dim % KVQ_BLOCK != 0)
    return fail(KVQ_ERR_ARG,
                "%s: head_dim %d is not a multiple of the %d-element quantization block", fn,
                head_dim, KVQ_BLOCK);
  if (dtype == KVQ_BF16 && head_dim % 8 != 0)
    return fail(KVQ_ERR_ARG, "%s: head_dim %d is not a multiple of 8", fn, head_dim);
  if (page_size < 1 || page_size > 1024)
    return fail(KVQ_ERR_ARG, "%s: page_size %d outside 1..1024", fn, page_size);
  if (dtype == KVQ_FP8_DS_MLA && !dsm_shape_ok(n_heads, head_dim))
    return fail(KVQ_ERR_UNSUPPORTED, "%s: the 656-byte row holds one head of 576 elements", fn);
  if (num_pages < 0) return fail(KVQ_ERR_ARG, "%s: num_pages < 0", fn);
  if (num_pages * (int64_t)page_size > INT32_MAX)
    return fail(KVQ_ERR_ARG, "%s: pool capacity exceeds 2^31-1 slots", fn);
  return KVQ_OK;
}

// The new tokens of a decode with append (kvq_paged_decode_append).
struct AppendIn {
  const void* new_k;
  const void* new_v;
  int64_t stride;  // elements between sequences
};

// The validation and launches of kvq_paged_decode; with use_scratch the
// workspace is the library's own array (kvq_paged_decode_noalloc), with app
// the call first appends each sequence's new token (kvq_paged_decode_append).
int decode_call(const char* fn, kvq_dtype dtype, const void* q, const void* k_pool,
                     const uint16_t* k_scales, const void* v_pool, const uint16_t* v_scales,
                     const int32_t* page_table, int64_t pt_stride, const int32_t* seq_lens,
                     const int32_t* seq_lens_host, int batch, int n_q_heads, int n_kv_heads,
                     int head_dim_qk, int head_dim_v, int page_size, int max_pages,
                     int64_t num_pages, float sm_scale, void* out_bf16, float* lse,
                     void* workspace, size_t workspace_bytes, kvq_stream_t stream,
                bool use_scratch, const AppendIn* app = nullptr) {
  if (!known_dtype(dtype)) return fail(KVQ_ERR_ARG, "%s: unknown dtype %d", fn, dtype);
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || max_pages < 1 || head_dim_qk < 1 ||
      head_dim_v < 1 || page_size < 1)
    return fail(KVQ_ERR_ARG, "%s: sizes must be >= 1", fn);
  if (n_q_heads % n_kv_heads != 0)
    return fail(KVQ_ERR_ARG, "%s: n_q_heads %d is not a multiple of n_kv_heads %d", fn,
                n_q_heads, n_kv_heads);
  if (dtype != KVQ_BF16 && (head_dim_qk % KVQ_BLOCK || head_dim_v % KVQ_BLOCK))
    return fail(KVQ_ERR_ARG,
                "%s: head_dim %d/%d is not a multiple of the %d-element block", fn,
                head_dim_qk, head_dim_v, KVQ_BLOCK);
  if (head_dim_v > head_dim_qk)
    return fail(KVQ_ERR_ARG, "%s: head_dim_v %d > head_dim_qk %d", fn, head_dim_v,
                head_dim_qk);
  if (pt_stride < max_pages)
    return fail(KVQ_ERR_ARG, "%s: pt_stride %lld < max_pages %d", fn,
                (long long)pt_stride, max_pages);
  if (num_pages < 1 || num_pages * (int64_t)page_size > INT32_MAX)
    return fail(KVQ_ERR_ARG, "%s: num_pages must be in 1..2^31/page_size", fn);
  if (!(sm_scale == sm_scale) || sm_scale == INFINITY || sm_scale == -INFINITY)
    return fail(KVQ_ERR_ARG, "%s: sm_scale is not finite", fn);
  if (!q || !k_pool || !v_pool || !page_table || !seq_lens || !out_bf16)
    return fail(KVQ_ERR_ARG, "%s: null pointer", fn);
  if (scaled(dtype) && (!k_scales || !v_scales))
    return fail(KVQ_ERR_ARG, "%s: null scales", fn);
  const bool shared = (k_pool == v_pool);
  if (shared != (k_scales == v_scales) && scaled(dtype))
    return fail(KVQ_ERR_ARG, "%s: k_pool == v_pool requires k_scales == v_scales", fn);
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out_bf16, 4))
    return fail(KVQ_ERR_ARG, "%s: q and pools must be 16-byte aligned", fn);
  kvq::DecodePlan plan;
  const char* why = nullptr;
  if (!kvq::plan_decode(dtype, batch, n_q_heads, n_kv_heads, head_dim_qk, head_dim_v, page_size,
                        max_pages, &plan, &why))
    return fail(KVQ_ERR_UNSUPPORTED, "%s: %s", fn, why);
  if (shared && plan.kind != kvq::DK_MLA)
    return fail(KVQ_ERR_UNSUPPORTED,
                "%s: k_pool == v_pool is only supported for the 576/512 slab", fn);
  if (!shared && plan.kind == kvq::DK_MLA)
    return fail(KVQ_ERR_UNSUPPORTED, "%s: the 576/512 shape needs the shared slab", fn);
  if (use_scratch) {  // the library's own array (kvq_paged_decode_noalloc)
    if (plan.bytes > kvq::scratch_bytes())
      return fail(KVQ_ERR_WORKSPACE,
                  "%s: these shapes need %zu bytes of scratch; the library's array holds %zu", fn,
                  plan.bytes, kvq::scratch_bytes());
    hipError_t e = kvq::scratch_pointer(&workspace);
    if (e != hipSuccess) return hip_fail(e, fn);
    workspace_bytes = kvq::scratch_bytes();
  }
  if (app) {
    if (!app->new_k) return fail(KVQ_ERR_ARG, "%s: null new_k", fn);
    if (shared != (app->new_v == nullptr))
      return fail(KVQ_ERR_ARG,
                  "%s: new_v must be null exactly when K and V share one slab (k_pool == v_pool)",
                  fn);
    if (app->stride < (int64_t)n_kv_heads * head_dim_qk || app->stride % 8 != 0)
      return fail(KVQ_ERR_ARG,
                  "%s: new_token_stride %lld must be >= n_kv_heads*head_dim_qk and a multiple of 8",
                  fn, (long long)app->stride);
    if (!aligned(app->new_k, 16) || (app->new_v && !aligned(app->new_v, 16)))
      return fail(KVQ_ERR_ARG, "%s: new_k/new_v must be 16-byte aligned", fn);
  }
  if (!workspace || workspace_bytes < plan.bytes)
    return fail(KVQ_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn,
                plan.bytes, workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256))
    return fail(KVQ_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  kvq::DecodeArgs a;
  a.qtype = dtype;
  a.q = static_cast<const uint16_t*>(q);
  a.k_pool = static_cast<const uint8_t*>(k_pool);
  a.k_scales = k_scales;
  a.v_pool = static_cast<const uint8_t*>(v_pool);
  a.v_scales = v_scales;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.head_dim_qk = head_dim_qk;
  a.head_dim_v = head_dim_v;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.sm_scale = sm_scale;
  a.out = static_cast<uint16_t*>(out_bf16);
  a.lse = lse;
  a.workspace = workspace;
  if (seq_lens_host) a.items_hint = host_items(plan, a, seq_lens_host);
  const int cus = num_cus_current();
  if (use_scratch) {
    // the array keeps the previous call's contents, whatever its shapes:
    // clear this plan's arrival counters (a fill kernel, no memset node)
    hipError_t z = kvq::launch_zero_words(static_cast<char*>(workspace) + plan.off_count,
                                          (plan.off_ml - plan.off_count) / 4, stream);
    if (z != hipSuccess) return hip_fail(z, fn);
  }
  const bool valu = plan.kind != kvq::DK_MLA && !plan.mfma;
  if (app && valu) {
    // the VALU kernel stores and attends the new token in the same launch
    a.new_kv[0] = static_cast<const uint16_t*>(app->new_k);
    a.new_kv[1] = static_cast<const uint16_t*>(app->new_v);
    a.new_stride = app->stride;
  } else if (app) {
    // the matrix-core and slab kernels: the append store, then the decode
    kvq::StoreArgs st;
    st.qtype = dtype;
    st.src[0] = static_cast<const uint16_t*>(app->new_k);
    st.src[1] = static_cast<const uint16_t*>(app->new_v);
    st.stride = app->stride;
    st.slots = nullptr;
    st.n_tokens = batch;
    st.n_heads = n_kv_heads;
    st.head_dim = head_dim_qk;
    st.page_size = page_size;
    st.num_pages = num_pages;
    st.pool[0] = static_cast<uint8_t*>(const_cast<void*>(k_pool));
    st.pool[1] = app->new_v ? static_cast<uint8_t*>(const_cast<void*>(v_pool)) : nullptr;
    st.scales[0] = const_cast<uint16_t*>(k_scales);
    st.scales[1] = app->new_v ? const_cast<uint16_t*>(v_scales) : nullptr;
    st.seq_lens = seq_lens;
    st.page_table = page_table;
    st.pt_stride = pt_stride;
    st.max_pages = max_pages;
    hipError_t se = kvq::launch_store(st, stream);
    if (se != hipSuccess) return hip_fail(se, fn);
  }
  hipError_t e = (plan.kind == kvq::DK_MLA) ? kvq::launch_mla_decode(a, plan, cus, stream)
                 : plan.mfma                 ? kvq::launch_gqa_mfma_decode(a, plan, cus, stream)
                                             : kvq::launch_gqa_decode(a, plan, cus, stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

}  // namespace

namespace kvq {

bool plan_decode(int qtype, int batch, int n_q_heads, int n_kv_heads, int head_dim_qk,
                 int head_dim_v, int page_size, int max_pages, DecodePlan* plan,
                 const char** why, int ext_new) {
  static thread_local char msg[256];
  auto no = [&](const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(msg, sizeof msg, fmt, ap);
    va_end(ap);
    *why = msg;
    return false;
  };
  if (!known_dtype(qtype)) return no("unknown dtype %d", qtype);
  if (batch < 1 || batch > kMaxBatch) return no("batch %d outside 1..%d", batch, kMaxBatch);
  if (n_kv_heads < 1 || n_q_heads < 1) return no("head counts must be >= 1");
  if (n_q_heads % n_kv_heads != 0)
    return no("n_q_heads %d is not a multiple of n_kv_heads %d", n_q_heads, n_kv_heads);
  if (max_pages < 1) return no("max_pages %d < 1", max_pages);
  if (page_size != kPageSize) return no("page_size %d is not supported (only 16)", page_size);
  if (qtype != KVQ_BF16 && (head_dim_qk % KVQ_BLOCK || head_dim_v % KVQ_BLOCK))
    return no("head_dim %d/%d is not a multiple of the %d-element quantization block",
              head_dim_qk, head_dim_v, KVQ_BLOCK);
  if (head_dim_v > head_dim_qk) return no("head_dim_v %d > head_dim_qk %d", head_dim_v, head_dim_qk);
  if (qtype == KVQ_FP8_DS_MLA &&
      !(head_dim_qk == kMlaDqk && head_dim_v == kMlaDv && n_kv_heads == 1 && ext_new == 0))
    return no("the 656-byte row is the decode format of the 576/512 slab only");
  DecodePlan p{};
  const int G = n_q_heads / n_kv_heads;
  if (ext_new > 0 && !(head_dim_qk == head_dim_v &&
                       (head_dim_qk == 64 || head_dim_qk == 128 || head_dim_qk == 256)))
    return no("extend attention needs separate K/V pools with head_dim 64, 128 or 256 (got "
              "%d/%d)", head_dim_qk, head_dim_v);
  if (ext_new > kExtendMaxNew) return no("max_new_tokens %d exceeds %d", ext_new, kExtendMaxNew);
  if (head_dim_qk == kMlaDqk && head_dim_v == kMlaDv && n_kv_heads == 1) {
    if (n_q_heads % 16 != 0 || n_q_heads > 128)
      return no("the 576/512 slab needs n_q_heads a multiple of 16 up to 128 (got %d)", n_q_heads);
    if (batch > kMlaMaxBatch)
      return no("batch %d exceeds %d for the 576/512 slab", batch, kMlaMaxBatch);
    p.kind = DK_MLA;
    p.gt = n_q_heads;
    p.n_hg = 1;
    // Item length in 32-token tiles: about one item per CU over the
    // upper-bound context, at most kMlaMaxItemPages pages.
    const int64_t tiles_per_seq = ((int64_t)max_pages * kPageSize + kMlaTile - 1) / kMlaTile;
    int64_t item_tiles = ((int64_t)batch * tiles_per_seq + kPlanCUs - 1) / kPlanCUs;
    const int64_t max_tiles = kMlaMaxItemPages * kPageSize / kMlaTile;
    if (item_tiles < 1) item_tiles = 1;
    if (item_tiles > max_tiles) item_tiles = max_tiles;
    p.item_pages = (int)(item_tiles * kMlaTile / kPageSize);
    const int64_t chunks = (max_pages + p.item_pages - 1) / p.item_pages;
    if (chunks > kMlaMaxChunks)
      return no("max_pages %d is too large for the 576/512 slab (at most %d)", max_pages,
                kMlaMaxChunks * kMlaMaxItemPages);
    p.fused_merge = false;
    p.max_items = (int64_t)batch * chunks;
  } else if (head_dim_qk == head_dim_v &&
             (head_dim_qk == 32 || head_dim_qk == 64 || head_dim_qk == 128 || head_dim_qk == 256)) {
    p.kind = DK_GQA;
    // 8 or more query heads per kv head (up to 16, or a multiple of 16) run
    // on the matrix-core kernel, the G heads as one padded 16-wide tile
    // Extend attention: the ext_new x G query rows of a kv head (token-major)
    // form ceil(rows / 16) tiles of up to 16 columns on the matrix cores.
    if (ext_new > 0) {
      const int64_t rows = (int64_t)ext_new * G;
      p.mfma = true;
      p.gt = rows <= 16 ? (int)rows : 16;
      // two full tiles per unit up to head_dim 128: every wave computes both
      // over its pages, so each page is loaded once for 32 query rows
      p.tn = (rows > 16 && head_dim_qk <= 128) ? 2 : 1;
      p.n_hg = (int)((rows + p.gt * p.tn - 1) / (p.gt * p.tn));
    } else {
      p.mfma = G >= 8 && head_dim_qk >= 64 && (G <= 16 || G % 16 == 0);
      if (p.mfma)
        p.gt = (G <= 16) ? G : 16;
      else
        p.gt = (G % 8 == 0) ? 8 : (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
      p.n_hg = G / p.gt;
    }
    const int64_t seq_units = (int64_t)n_kv_heads * p.n_hg;  // (kv head, head group) pairs
    const int64_t units = (int64_t)batch * seq_units;
    // Work items are sized on the device from the actual lengths (about
    // `target` of them over the batch, one per resident workgroup); here only
    // the bounds: whole steps of pages per wave, at most kMaxItemPages, and
    // few enough chunks per sequence for the merge's weights to fit in LDS.
    const int step = kDecodeWaves * (p.mfma ? 1 : gqa_pages_per_step(qtype, head_dim_qk) * kGqaDepth);
    // one item per CU; extend attention (many more query rows) two
    const int64_t target = (p.mfma && ext_new > 0 ? 2 : 1) * (int64_t)kPlanCUs;
    const int cap = kMaxItemPages / step * step;
    // The split plan: items of at most `cap` pages, at least `min_pages`.
    const int64_t for_merge =
        ((int64_t)max_pages * p.gt * p.tn + kMergeMaxWeights - 1) / kMergeMaxWeights;
    int64_t min_pages = ((for_merge > step ? for_merge : step) + step - 1) / step * step;
    // the in-kernel merge holds chunks x columns weights in LDS, and a
    // sequence splits into ceil(max_pages / item pages) chunks: rounding up
    // can add one chunk past max_pages * columns / kMergeMaxWeights when the
    // column count does not divide kMergeMaxWeights (12 columns: 342 x 12)
    while (min_pages <= cap &&
           (max_pages + min_pages - 1) / min_pages * p.gt * p.tn > kMergeMaxWeights)
      min_pages += step;
    const bool split_ok = min_pages <= cap;
    // items: at most work / item_pages + one partial item per (sequence, unit);
    // item_pages >= work / target unless capped, and >= min_pages always
    int64_t split_items = 0;
    if (split_ok) {
      const int64_t by_min = units * ((max_pages + min_pages - 1) / min_pages);
      int64_t by_target = ((int64_t)batch * max_pages * seq_units + cap - 1) / cap;
      if (by_target < target) by_target = target;
      by_target += units;
      split_items = by_min < by_target ? by_min : by_target;
    }
    const double split_partials =
        (double)split_items * p.gt * p.tn * (2 + head_dim_v) * sizeof(float);
    if (ext_new > 0 && units >= kWholeUnitsPerWorkgroup * target &&
        (!split_ok || split_partials > (double)kWholeMinPartialBytes)) {
      // Long prefill whose split-K partials would be huge: each (sequence,
      // unit) is one item over the whole sequence (the kernel streams it in
      // sub-chunks of kMaxItemPages), so nothing splits and the workspace
      // holds no partials.  (Slower than the split plan where both fit:
      // 1892 against 1428 us for 512 new tokens of 8 x 16384.)
      const int whole = (int)((max_pages + step - 1) / step * step);
      p.whole = true;
      p.step = step;
      p.min_pages = whole;
      p.cap_pages = whole;
      p.target = (int)target;
      p.item_pages = whole;
      p.max_items = units;
      p.fused_merge = true;
    } else {
      if (!split_ok) return no("max_pages %d is too large for the split-K merge", max_pages);
      p.step = step;
      p.min_pages = (int)min_pages;
      p.cap_pages = cap;
      p.target = (int)target;
      p.item_pages = (int)min_pages;
      p.max_items = split_items;
      // chunks of one sequence: at most max_pages / min_pages, and at most
      // about target / seq_units unless the item size is capped
      int64_t chunks = (max_pages + cap - 1) / cap;
      if (chunks < target / seq_units + 1) chunks = target / seq_units + 1;
      if (chunks > (max_pages + min_pages - 1) / min_pages) chunks = (max_pages + min_pages - 1) / min_pages;
      // the last workgroup merges a sequence's partials itself while they are
      // small; beyond that a merge kernel spreads the reads over the GPU
      // (extend attention: many tiles per sequence, so items rarely split; a
      // merge kernel would launch a block per output row only to find one
      // chunk)
      p.fused_merge = ext_new > 0 || head_dim_v < 64 ||
                      chunks * p.gt * head_dim_v * (int64_t)sizeof(float) <= kFusedMergeMaxBytes;
    }
  } else {
    return no("head_dim %d/%d is not supported (separate K/V: 32, 64, 128 or 256 with equal "
              "K and V widths; shared slab: 576/512 with one kv head)",
              head_dim_qk, head_dim_v);
  }
  if (p.max_items >= ((int64_t)1 << 31)) return no("too many work items");
  p.off_prefix = 0;
  p.off_count = align256((size_t)(batch + 1) * sizeof(int));
  p.off_ml = p.off_count + align256((size_t)batch * n_kv_heads * p.n_hg * sizeof(int));
  // split-K partials (none when no item splits)
  const size_t parts = p.whole ? 0 : (size_t)p.max_items;
  p.off_acc = p.off_ml + align256(parts * p.gt * p.tn * 2 * sizeof(float));
  // split-K partial outputs: fp32 accumulators (GQA) or bf16 normalized rows (MLA)
  const size_t acc_elem = (p.kind == DK_MLA) ? sizeof(uint16_t) : sizeof(float);
  p.bytes = p.off_acc + align256(parts * p.gt * p.tn * head_dim_v * acc_elem);
  *plan = p;
  return true;
}

bool plan_sparse(int qtype, int batch, int n_q_heads, int k, SparseLayout* lay,
                 const char** why) {
  static thread_local char msg[256];
  if (k < 1 || k > kSparseMaxK) {
    snprintf(msg, sizeof msg, "top-k count %d outside 1..%d", k, kSparseMaxK);
    *why = msg;
    return false;
  }
  // The slab decode plans over the lists as sequences of k entries (k
  // rounded up to whole pages): item size, item count and the split-K
  // partials, which are all the workspace holds.
  SparseLayout L{};
  L.kk = (k + kPageSize - 1) / kPageSize * kPageSize;
  if (!plan_decode(qtype, batch, n_q_heads, 1, kMlaDqk, kMlaDv, kPageSize, L.kk / kPageSize,
                   &L.dense, why))
    return false;
  L.bytes = L.dense.bytes;
  *lay = L;
  return true;
}

}  // namespace kvq

extern "C" {

const char* kvq_last_error(void) { return g_err.c_str(); }

int64_t kvq_pool_bytes(kvq_dtype dtype, int64_t num_pages, int page_size, int n_heads,
                       int head_dim, int64_t* scale_bytes) {
  if (!known_dtype(dtype)) return fail(-1, "kvq_pool_bytes: unknown dtype %d", (int)dtype);
  if (num_pages < 0 || page_size < 1 || n_heads < 1 || head_dim < 1)
    return fail(-1, "kvq_pool_bytes: sizes must be positive (num_pages may be 0)");
  if (dtype != KVQ_BF16 && head_dim % KVQ_BLOCK != 0)
    return fail(-1, "kvq_pool_bytes: head_dim %d is not a multiple of %d", head_dim, KVQ_BLOCK);
  if (dtype == KVQ_FP8_DS_MLA && !dsm_shape_ok(n_heads, head_dim))
    return fail(-1, "kvq_pool_bytes: the 656-byte row holds one head of 576 elements");
  const int64_t elems = num_pages * page_size * (int64_t)n_heads * head_dim;
  const int64_t codes = (dtype == KVQ_BF16)         ? 2 * elems
                        : (dtype == KVQ_FP8_DS_MLA) ? num_pages * page_size * (int64_t)kvq::kDsmRow
                                                    : elems;
  const int64_t scales = scaled(dtype) ? (elems / KVQ_BLOCK) * 2 : 0;
  if (scale_bytes) *scale_bytes = scales;
  g_err.clear();
  return codes + scales;
}

int kvq_store(kvq_dtype dtype, const void* k_src, const void* v_src, int64_t src_token_stride,
              const int32_t* slot_mapping, int64_t n_tokens, int n_heads, int head_dim,
              int page_size, int64_t num_pages, void* k_pool, uint16_t* k_scales, void* v_pool,
              uint16_t* v_scales, kvq_stream_t stream) {
  int rc = check_rows(dtype, n_tokens, n_heads, head_dim, page_size, num_pages, "kvq_store");
  if (rc != KVQ_OK) return rc;
  if (n_tokens == 0) return ok();
  if (!k_src || !slot_mapping || !k_pool) return fail(KVQ_ERR_ARG, "kvq_store: null pointer");
  if (scaled(dtype) && !k_scales) return fail(KVQ_ERR_ARG, "kvq_store: null k_scales");
  if (v_src && (!v_pool || (scaled(dtype) && !v_scales)))
    return fail(KVQ_ERR_ARG, "kvq_store: v_src given without v_pool/v_scales");
  if (v_src && dtype == KVQ_FP8_DS_MLA)
    return fail(KVQ_ERR_ARG, "kvq_store: the 656-byte row is one slab (K and V the same row)");
  if (src_token_stride < (int64_t)n_heads * head_dim || src_token_stride % 8 != 0)
    return fail(KVQ_ERR_ARG,
                "kvq_store: src_token_stride %lld must be >= n_heads*head_dim and a multiple of 8",
                (long long)src_token_stride);
  if (!aligned(k_src, 16) || (v_src && !aligned(v_src, 16)))
    return fail(KVQ_ERR_ARG, "kvq_store: k_src/v_src must be 16-byte aligned");
  if (!aligned(k_pool, 16) || (v_src && !aligned(v_pool, 16)))
    return fail(KVQ_ERR_ARG, "kvq_store: pools must be 16-byte aligned");
  if (scaled(dtype) && (!aligned(k_scales, 2) || (v_src && !aligned(v_scales, 2))))
    return fail(KVQ_ERR_ARG, "kvq_store: scales must be 2-byte aligned");
  kvq::StoreArgs a;
  a.qtype = dtype;
  a.src[0] = static_cast<const uint16_t*>(k_src);
  a.src[1] = static_cast<const uint16_t*>(v_src);
  a.stride = src_token_stride;
  a.slots = slot_mapping;
  a.n_tokens = n_tokens;
  a.n_heads = n_heads;
  a.head_dim = head_dim;
  a.page_size = page_size;
  a.num_pages = num_pages;
  a.pool[0] = static_cast<uint8_t*>(k_pool);
  a.pool[1] = static_cast<uint8_t*>(v_src ? v_pool : nullptr);
  a.scales[0] = k_scales;
  a.scales[1] = v_src ? v_scales : nullptr;
  hipError_t e = kvq::launch_store(a, stream);
  if (e != hipSuccess) return hip_fail(e, "kvq_store");
  return ok();
}

int kvq_dequant(kvq_dtype dtype, const void* pool, const uint16_t* scales,
                const int32_t* slot_mapping, int64_t n_tokens, int n_heads, int head_dim,
                int page_size, int64_t num_pages, void* out_bf16, kvq_stream_t stream) {
  int rc = check_rows(dtype, n_tokens, n_heads, head_dim, page_size, num_pages, "kvq_dequant");
  if (rc != KVQ_OK) return rc;
  if (n_tokens == 0) return ok();
  if (!pool || !slot_mapping || !out_bf16 || (scaled(dtype) && !scales))
    return fail(KVQ_ERR_ARG, "kvq_dequant: null pointer");
  if (!aligned(pool, 16) || !aligned(out_bf16, 16))
    return fail(KVQ_ERR_ARG, "kvq_dequant: pool and out must be 16-byte aligned");
  kvq::DequantArgs a;
  a.qtype = dtype;
  a.pool = static_cast<const uint8_t*>(pool);
  a.scales = scales;
  a.slots = slot_mapping;
  a.n_tokens = n_tokens;
  a.n_heads = n_heads;
  a.head_dim = head_dim;
  a.page_size = page_size;
  a.num_pages = num_pages;
  a.out = static_cast<uint16_t*>(out_bf16);
  hipError_t e = kvq::launch_dequant(a, stream);
  if (e != hipSuccess) return hip_fail(e, "kvq_dequant");
  return ok();
}

size_t kvq_paged_decode_workspace_bytes(int batch, int n_q_heads, int n_kv_heads,
                                        int head_dim_v, int max_pages, int page_size) {
  // The shapes fix the kernel: one kv head with a 512-wide V is the 576/512
  // slab, anything else has K as wide as V.  The storage type only changes
  // how finely items may split, so the answer covers every type.
  const int head_dim_qk =
      (n_kv_heads == 1 && head_dim_v == kvq::kMlaDv) ? kvq::kMlaDqk : head_dim_v;
  size_t need = 0;
  const char* why = nullptr;
  for (int dtype : {KVQ_BF16, KVQ_FP8_E4M3, KVQ_Q8_0, KVQ_FP8_E4M3_CAST, KVQ_FP8_E5M2_CAST,
                    KVQ_FP8_DS_MLA}) {
    kvq::DecodePlan p;
    const char* w = nullptr;
    if (kvq::plan_decode(dtype, batch, n_q_heads, n_kv_heads, head_dim_qk, head_dim_v, page_size,
                         max_pages, &p, &w)) {
      if (p.bytes > need) need = p.bytes;
    } else if (!why) {
      why = w;
    }
  }
  if (need == 0) {
    fail(KVQ_ERR_UNSUPPORTED, "kvq_paged_decode_workspace_bytes: %s", why);
    return 0;
  }
  g_err.clear();
  return need;
}

int kvq_paged_decode(kvq_dtype dtype, const void* q, const void* k_pool,
                     const uint16_t* k_scales, const void* v_pool, const uint16_t* v_scales,
                     const int32_t* page_table, int64_t pt_stride, const int32_t* seq_lens,
                     const int32_t* seq_lens_host, int batch, int n_q_heads, int n_kv_heads,
                     int head_dim_qk, int head_dim_v, int page_size, int max_pages,
                     int64_t num_pages, float sm_scale, void* out_bf16, float* lse,
                     void* workspace, size_t workspace_bytes, kvq_stream_t stream) {
  return decode_call("kvq_paged_decode", dtype, q, k_pool, k_scales, v_pool, v_scales, page_table,
                     pt_stride, seq_lens, seq_lens_host, batch, n_q_heads, n_kv_heads,
                     head_dim_qk, head_dim_v, page_size, max_pages, num_pages, sm_scale, out_bf16,
                     lse, workspace, workspace_bytes, stream, false);
}

int kvq_paged_decode_noalloc(kvq_dtype dtype, const void* q, const void* k_pool,
                             const uint16_t* k_scales, const void* v_pool,
                             const uint16_t* v_scales, const int32_t* page_table,
                             int64_t pt_stride, const int32_t* seq_lens,
                             const int32_t* seq_lens_host, int batch, int n_q_heads,
                             int n_kv_heads, int head_dim_qk, int head_dim_v, int page_size,
                             int max_pages, int64_t num_pages, float sm_scale, void* out_bf16,
                             float* lse, kvq_stream_t stream) {
  return decode_call("kvq_paged_decode_noalloc", dtype, q, k_pool, k_scales, v_pool, v_scales,
                     page_table, pt_stride, seq_lens, seq_lens_host, batch, n_q_heads, n_kv_heads,
                     head_dim_qk, head_dim_v, page_size, max_pages, num_pages, sm_scale, out_bf16,
                     lse, nullptr, 0, stream, true);
}

int kvq_paged_decode_append(kvq_dtype dtype, const void* q, const void* new_k,
                            const void* new_v, int64_t new_token_stride, void* k_pool,
                            uint16_t* k_scales, void* v_pool, uint16_t* v_scales,
                            const int32_t* page_table, int64_t pt_stride, const int32_t* seq_lens,
                            const int32_t* seq_lens_host, int batch, int n_q_heads,
                            int n_kv_heads, int head_dim_qk, int head_dim_v, int page_size,
                            int max_pages, int64_t num_pages, float sm_scale, void* out_bf16,
                            float* lse, void* workspace, size_t workspace_bytes,
                            kvq_stream_t stream) {
  const AppendIn app{new_k, new_v, new_token_stride};
  return decode_call("kvq_paged_decode_append", dtype, q, k_pool, k_scales, v_pool, v_scales,
                     page_table, pt_stride, seq_lens, seq_lens_host, batch, n_q_heads, n_kv_heads,
                     head_dim_qk, head_dim_v, page_size, max_pages, num_pages, sm_scale, out_bf16,
                     lse, workspace, workspace_bytes, stream, false, &app);
}

size_t kvq_extend_attention_workspace_bytes(kvq_dtype dtype, int batch, int n_q_heads,
                                            int n_kv_heads, int head_dim, int page_size,
                                            int max_pages, int max_new_tokens) {
  kvq::DecodePlan p;
  const char* why = nullptr;
  if (max_new_tokens < 1) {
    fail(KVQ_ERR_ARG, "kvq_extend_attention_workspace_bytes: max_new_tokens must be >= 1");
    return 0;
  }
  const bool slab = head_dim == kvq::kMlaDqk && n_kv_heads == 1;
  if (slab && (int64_t)batch * max_new_tokens > kvq::kMlaMaxBatch) {
    fail(KVQ_ERR_UNSUPPORTED, "kvq_extend_attention_workspace_bytes: batch x max_new_tokens "
                              "exceeds %d for the 576/512 slab", kvq::kMlaMaxBatch);
    return 0;
  }
  if (!(slab ? kvq::plan_decode(dtype, batch * max_new_tokens, n_q_heads, 1, kvq::kMlaDqk,
                                kvq::kMlaDv, page_size, max_pages, &p, &why)
             : kvq::plan_decode(dtype, batch, n_q_heads, n_kv_heads, head_dim, head_dim,
                                page_size, max_pages, &p, &why, max_new_tokens))) {
    fail(KVQ_ERR_UNSUPPORTED, "kvq_extend_attention_workspace_bytes: %s", why);
    return 0;
  }
  g_err.clear();
  return p.bytes;
}

int kvq_extend_attention(kvq_dtype dtype, const void* q, const int32_t* q_start,
                         int max_new_tokens, const void* k_pool, const uint16_t* k_scales,
                         const void* v_pool, const uint16_t* v_scales, const int32_t* page_table,
                         int64_t pt_stride, const int32_t* seq_lens, int batch, int n_q_heads,
                         int n_kv_heads, int head_dim, int page_size, int max_pages,
                         int64_t num_pages, float sm_scale, void* out_bf16, float* lse,
                         void* workspace, size_t workspace_bytes, kvq_stream_t stream) {
  if (!known_dtype(dtype))
    return fail(KVQ_ERR_ARG, "kvq_extend_attention: unknown dtype %d", dtype);
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || max_pages < 1 || head_dim < 1 ||
      page_size < 1 || max_new_tokens < 1)
    return fail(KVQ_ERR_ARG, "kvq_extend_attention: sizes must be >= 1");
  if (n_q_heads % n_kv_heads != 0)
    return fail(KVQ_ERR_ARG, "kvq_extend_attention: n_q_heads %d is not a multiple of n_kv_heads %d",
                n_q_heads, n_kv_heads);
  if (dtype != KVQ_BF16 && head_dim % KVQ_BLOCK)
    return fail(KVQ_ERR_ARG, "kvq_extend_attention: head_dim %d is not a multiple of the %d-element block",
                head_dim, KVQ_BLOCK);
  if (pt_stride < max_pages)
    return fail(KVQ_ERR_ARG, "kvq_extend_attention: pt_stride %lld < max_pages %d",
                (long long)pt_stride, max_pages);
  if (num_pages < 1 || num_pages * (int64_t)page_size > INT32_MAX)
    return fail(KVQ_ERR_ARG, "kvq_extend_attention: num_pages must be in 1..2^31/page_size");
  if (!(sm_scale == sm_scale) || sm_scale == INFINITY || sm_scale == -INFINITY)
    return fail(KVQ_ERR_ARG, "kvq_extend_attention: sm_scale is not finite");
  if (!q || !q_start || !k_pool || !v_pool || !page_table || !seq_lens || !out_bf16)
    return fail(KVQ_ERR_ARG, "kvq_extend_attention: null pointer");
  if (scaled(dtype) && (!k_scales || !v_scales))
    return fail(KVQ_ERR_ARG, "kvq_extend_attention: null scales");
  // the shared 576/512 slab: the MLA kernel with its work numbered by new token
  const bool slab = k_pool == v_pool;
  if (slab && !(head_dim == kvq::kMlaDqk && n_kv_heads == 1 && k_scales == v_scales))
    return fail(KVQ_ERR_UNSUPPORTED,
                "kvq_extend_attention: k_pool == v_pool is the 576/512 slab (one kv head, "
                "the same scales)");
  if (!slab && (head_dim == kvq::kMlaDqk || dtype == KVQ_FP8_DS_MLA))
    return fail(KVQ_ERR_UNSUPPORTED, "kvq_extend_attention: the 576-wide slab needs k_pool == v_pool");
  if (slab && (int64_t)batch * max_new_tokens > kvq::kMlaMaxBatch)
    return fail(KVQ_ERR_UNSUPPORTED,
                "kvq_extend_attention: batch x max_new_tokens exceeds %d for the 576/512 slab",
                kvq::kMlaMaxBatch);
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out_bf16, 4))
    return fail(KVQ_ERR_ARG, "kvq_extend_attention: q and pools must be 16-byte aligned");
  kvq::DecodePlan plan;
  const char* why = nullptr;
  if (!(slab ? kvq::plan_decode(dtype, batch * max_new_tokens, n_q_heads, 1, kvq::kMlaDqk,
                                kvq::kMlaDv, page_size, max_pages, &plan, &why)
             : kvq::plan_decode(dtype, batch, n_q_heads, n_kv_heads, head_dim, head_dim,
                                page_size, max_pages, &plan, &why, max_new_tokens)))
    return fail(KVQ_ERR_UNSUPPORTED, "kvq_extend_attention: %s", why);
  if (!workspace || workspace_bytes < plan.bytes)
    return fail(KVQ_ERR_WORKSPACE, "kvq_extend_attention: workspace of %zu bytes needed, %zu given",
                plan.bytes, workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256))
    return fail(KVQ_ERR_WORKSPACE, "kvq_extend_attention: workspace must be 256-byte aligned");
  kvq::DecodeArgs a;
  a.qtype = dtype;
  a.q = static_cast<const uint16_t*>(q);
  a.k_pool = static_cast<const uint8_t*>(k_pool);
  a.k_scales = k_scales;
  a.v_pool = static_cast<const uint8_t*>(v_pool);
  a.v_scales = v_scales;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.head_dim_qk = head_dim;
  a.head_dim_v = head_dim;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.sm_scale = sm_scale;
  a.out = static_cast<uint16_t*>(out_bf16);
  a.lse = lse;
  a.workspace = workspace;
  a.q_start = q_start;
  a.max_new = max_new_tokens;
  if (slab) {  // work index v = b * max_new + i over the new tokens
    a.batch = batch * max_new_tokens;
    a.head_dim_v = kvq::kMlaDv;
  }
  hipError_t e = slab ? kvq::launch_mla_decode(a, plan, num_cus_current(), stream)
                      : kvq::launch_gqa_mfma_decode(a, plan, num_cus_current(), stream);
  if (e != hipSuccess) return hip_fail(e, "kvq_extend_attention");
  return ok();
}

size_t kvq_sparse_mla_decode_workspace_bytes(kvq_dtype dtype, int batch, int n_q_heads,
                                             int topk) {
  kvq::SparseLayout lay;
  const char* why = nullptr;
  if (!kvq::plan_sparse(dtype, batch, n_q_heads, topk, &lay, &why)) {
    fail(KVQ_ERR_UNSUPPORTED, "kvq_sparse_mla_decode_workspace_bytes: %s", why);
    return 0;
  }
  g_err.clear();
  return lay.bytes;
}

int kvq_sparse_mla_decode(kvq_dtype dtype, const void* q, const void* slab,
                          const uint16_t* scales, const int32_t* page_table, int64_t pt_stride,
                          const int32_t* seq_lens, const int32_t* topk_idx, int64_t topk_stride,
                          int topk, int batch, int n_q_heads, int page_size, int max_pages,
                          int64_t num_pages, float sm_scale, void* out_bf16, float* lse,
                          void* workspace, size_t workspace_bytes, kvq_stream_t stream) {
  if (!known_dtype(dtype))
    return fail(KVQ_ERR_ARG, "kvq_sparse_mla_decode: unknown dtype %d", dtype);
  if (batch < 1 || n_q_heads < 1 || max_pages < 1 || page_size < 1 || topk < 1)
    return fail(KVQ_ERR_ARG, "kvq_sparse_mla_decode: sizes must be >= 1");
  if (topk_stride < topk)
    return fail(KVQ_ERR_ARG, "kvq_sparse_mla_decode: topk_stride %lld < topk %d",
                (long long)topk_stride, topk);
  if (pt_stride < max_pages)
    return fail(KVQ_ERR_ARG, "kvq_sparse_mla_decode: pt_stride %lld < max_pages %d",
                (long long)pt_stride, max_pages);
  if (page_size != kvq::kPageSize)
    return fail(KVQ_ERR_UNSUPPORTED, "kvq_sparse_mla_decode: page_size %d is not supported",
                page_size);
  if (num_pages < 1 || num_pages * (int64_t)page_size > INT32_MAX)
    return fail(KVQ_ERR_ARG, "kvq_sparse_mla_decode: num_pages must be in 1..2^31/page_size");
  if (!(sm_scale == sm_scale) || sm_scale == INFINITY || sm_scale == -INFINITY)
    return fail(KVQ_ERR_ARG, "kvq_sparse_mla_decode: sm_scale is not finite");
  if (!q || !slab || !page_table || !seq_lens || !topk_idx || !out_bf16 ||
      (scaled(dtype) && !scales))
    return fail(KVQ_ERR_ARG, "kvq_sparse_mla_decode: null pointer");
  if (!aligned(q, 16) || !aligned(slab, 16) || !aligned(out_bf16, 4) ||
      (scaled(dtype) && !aligned(scales, 4)))
    return fail(KVQ_ERR_ARG, "kvq_sparse_mla_decode: q and slab must be 16-byte aligned, "
                             "scales 4-byte aligned");
  kvq::SparseLayout lay;
  const char* why = nullptr;
  if (!kvq::plan_sparse(dtype, batch, n_q_heads, topk, &lay, &why))
    return fail(KVQ_ERR_UNSUPPORTED, "kvq_sparse_mla_decode: %s", why);
  if (!workspace || workspace_bytes < lay.bytes)
    return fail(KVQ_ERR_WORKSPACE, "kvq_sparse_mla_decode: workspace of %zu bytes needed, %zu given",
                lay.bytes, workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256))
    return fail(KVQ_ERR_WORKSPACE, "kvq_sparse_mla_decode: workspace must be 256-byte aligned");
  kvq::DecodeArgs a;
  a.qtype = dtype;
  a.q = static_cast<const uint16_t*>(q);
  a.k_pool = a.v_pool = static_cast<const uint8_t*>(slab);
  a.k_scales = a.v_scales = scaled(dtype) ? scales : nullptr;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = 1;
  a.head_dim_qk = kvq::kMlaDqk;
  a.head_dim_v = kvq::kMlaDv;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.sm_scale = sm_scale;
  a.out = static_cast<uint16_t*>(out_bf16);
  a.lse = lse;
  a.workspace = workspace;
  a.topk = topk_idx;
  a.topk_stride = topk_stride;
  a.topk_k = topk;
  hipError_t e = kvq::launch_mla_decode(a, lay.dense, num_cus_current(), stream);
  if (e != hipSuccess) return hip_fail(e, "kvq_sparse_mla_decode");
  return ok();
}

int kvq_debug_e4m3_encode_range(uint32_t first_bits, int64_t count, uint8_t* out_codes,
                                kvq_stream_t stream) {
  if (count < 0 || count % 4 != 0 || (int64_t)first_bits + count > ((int64_t)1 << 32))
    return fail(KVQ_ERR_ARG, "kvq_debug_e4m3_encode_range: count %lld must be a multiple of 4 "
                             "within the 2^32 bit patterns", (long long)count);
  if (count == 0) return ok();
  if (!out_codes || !aligned(out_codes, 4))
    return fail(KVQ_ERR_ARG, "kvq_debug_e4m3_encode_range: out_codes null or not 4-byte aligned");
  hipError_t e = kvq::launch_debug_e4m3(first_bits, count, out_codes, stream);
  if (e != hipSuccess) return hip_fail(e, "kvq_debug_e4m3_encode_range");
  return ok();
}

int kvq_debug_decode_plan(kvq_dtype dtype, int batch, int n_q_heads, int n_kv_heads,
                          int head_dim_qk, int head_dim_v, int max_pages, int max_new_tokens,
                          int64_t* out, int n_out) {
  kvq::DecodePlan p;
  const char* why = nullptr;
  if (!kvq::plan_decode(dtype, batch, n_q_heads, n_kv_heads, head_dim_qk, head_dim_v,
                        kvq::kPageSize, max_pages, &p, &why, max_new_tokens > 0 ? max_new_tokens : 0))
    return fail(KVQ_ERR_UNSUPPORTED, "kvq_debug_decode_plan: %s", why);
  const int64_t v[] = {p.kind, p.gt, p.tn, p.n_hg, p.step, p.min_pages, p.cap_pages, p.target,
                       p.max_items, (int64_t)p.bytes, p.item_pages, p.fused_merge ? 1 : 0,
                       p.mfma ? 1 : 0, p.whole ? 1 : 0};
  const int n = (int)(sizeof v / sizeof v[0]);
  int k = 0;
  for (; out && k < n_out && k < n; ++k) out[k] = v[k];
  g_err.clear();
  return k;
}

}  // extern "C"
