// kvq_sparse.hip -- sparse top-k decode over the shared MLA slab (gfx950):
// the listed rows are gathered into a compact slab, which the slab decode
// kernel (kvq_mla.hip) then attends to in full.
//
// Sources: [PR25] "Experimental FP8 KV Cache" (SPARSE_MLA_DECODE: D=576,
// Hq=128, Hkv=1, Dv=512, K=256 tokens selected out of the cache per query);
// [PR113] "feat(kvcache): 8-bit DSV4 window/compressed KV behind
// --kv-cache-dtype" (§What this adds: one slab, K and V the same row;
// §Testing: masked (-1) columns).
//
// Softmax attention over a set of rows does not depend on their order, so
// attending to the listed rows equals attending, in full, to a sequence made
// of exactly those rows.  An entry is taken when it is a position below the
// sequence's length on a page that is present; taken entries keep their list
// order and get consecutive places in the compact sequence.  Each list is cut
// into slices of 64 entries, one workgroup per slice: the workgroup counts the
// taken entries before its slice itself (no workgroup waits for another),
// places its own with one ballot, then copies their code rows (16-byte moves,
// every load of a thread issued before its first store) and scale rows into
// the workspace.  The first slice's workgroup writes the compact sequence's
// identity page table, the last one its length.  The codes are moved, not
// decoded, so the decode sees exactly the stored rows.
#include "kvq_attn.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kSlice = 64;  // list entries per workgroup: one wave's ballot

struct GatherArgs {
  const int32_t* topk;
  int64_t topk_stride;
  int k, kk;  // entries per list, and rows per compact sequence (k rounded up to a page)
  int slices; // workgroups per list
  const int32_t* page_table;
  int64_t pt_stride;
  const int32_t* seq_lens;
  int max_pages;
  int64_t num_pages;
  const uint8_t* slab;      // rows of row_bytes
  const uint16_t* scales;   // rows of kNB fp16, or null
  int row_bytes;
  uint8_t* g_slab;          // [batch * kk] rows
  uint16_t* g_scales;       // [batch * kk][kNB], or null
  int32_t* g_pt;            // [batch][kk / page]
  int32_t* g_len;           // [batch]
};

constexpr int kNB = kMlaDqk / 32;  // scales per row
constexpr int kScalePerThread = (kSlice * (kNB / 2) + kThreads - 1) / kThreads;

// Slot of list entry i of sequence b in the slab, or -1 when it is skipped.
__device__ __forceinline__ int64_t entry_slot(const GatherArgs& g, int b, int64_t L, int i) {
  if (i >= g.k) return -1;
  const int64_t t = g.topk[(int64_t)b * g.topk_stride + i];
  if (t < 0 || t >= L) return -1;
  const int64_t page = g.page_table[(int64_t)b * g.pt_stride + t / kPageSize];
  if (page < 0 || page >= g.num_pages) return -1;
  return page * kPageSize + t % kPageSize;
}

// kUnits: 16-byte moves per row (36 for 8-bit codes, 72 for bf16).
template <int kUnits>
__global__ __launch_bounds__(kThreads) void sparse_gather_kernel(GatherArgs g) {
  constexpr int kPerThread = (kSlice * kUnits + kThreads - 1) / kThreads;
  constexpr int kRowBytes = kUnits * 16;
  __shared__ int64_t s_src[kSlice];
  __shared__ int s_wave[kThreads / 64];
  __shared__ int s_own;
  const int b = blockIdx.x / g.slices, sl = blockIdx.x - b * g.slices;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t L = g.seq_lens[b];
  const int64_t cap = (int64_t)g.max_pages * kPageSize;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int start = sl * kSlice;
  // wave 0 places this slice's entries; every thread counts entries before it
  if (wave == 0) {
    const int64_t src = entry_slot(g, b, L, start + lane);
    const uint64_t m = __builtin_amdgcn_ballot_w64(src >= 0);
    if (src >= 0) s_src[__builtin_popcountll(m & ((1ull << lane) - 1ull))] = src;
    if (lane == 0) s_own = __builtin_popcountll(m);
  }
  int before = 0;
  for (int i = tid; i < start; i += kThreads) before += entry_slot(g, b, L, i) >= 0 ? 1 : 0;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) before += __shfl_xor(before, o, 64);
  if (lane == 0) s_wave[wave] = before;
  __syncthreads();
  int prefix = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) prefix += s_wave[w];
  const int n = s_own;
  const int64_t dst0 = (int64_t)b * g.kk + prefix;
  // Code rows: every load of a thread first, then the stores.  The slice's
  // rows land contiguously, so a move's offset in the destination is its
  // index times 16; an index past the slice's rows reads the slice's first
  // row again and its store falls outside the destination's buffer
  // descriptor, which drops it.  No load or store sits under a branch.
  if (n > 0) {
    const auto dst = page_rsrc(g.g_slab + dst0 * kRowBytes, n * kRowBytes);
    u32x4 v[kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      int u = tid + j * kThreads;
      u = u < n * kUnits ? u : 0;
      const int r = u / kUnits, c = u - r * kUnits;
      v[j] = *reinterpret_cast<const u32x4*>(g.slab + s_src[r] * kRowBytes + c * 16);
    }
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
      __builtin_amdgcn_raw_buffer_store_b128(v[j], dst, (tid + j * kThreads) * 16, 0, 0);
    if (g.scales) {  // two fp16 per move
      const auto sdst = page_rsrc(g.g_scales + dst0 * kNB, n * kNB * 2);
      uint32_t w[kScalePerThread];
#pragma unroll
      for (int j = 0; j < kScalePerThread; ++j) {
        int u = tid + j * kThreads;
        u = u < n * (kNB / 2) ? u : 0;
        const int r = u / (kNB / 2), c = u - r * (kNB / 2);
        w[j] = *reinterpret_cast<const uint32_t*>(g.scales + s_src[r] * kNB + 2 * c);
      }
#pragma unroll
      for (int j = 0; j < kScalePerThread; ++j)
        __builtin_amdgcn_raw_buffer_store_b32(w[j], sdst, (tid + j * kThreads) * 4, 0, 0);
    }
  }
  if (sl == 0) {
    const int gpages = g.kk / kPageSize;
    for (int p = tid; p < gpages; p += kThreads) g.g_pt[(int64_t)b * gpages + p] = b * gpages + p;
  }
  if (sl == g.slices - 1 && tid == 0) g.g_len[b] = prefix + n;
}

}  // namespace

hipError_t launch_sparse_gather(const SparseArgs& s, const SparseLayout& lay, int batch,
                                hipStream_t stream) {
  GatherArgs g;
  g.topk = s.topk;
  g.topk_stride = s.topk_stride;
  g.k = s.k;
  g.kk = lay.kk;
  g.slices = (s.k + kSlice - 1) / kSlice;
  g.page_table = s.page_table;
  g.pt_stride = s.pt_stride;
  g.seq_lens = s.seq_lens;
  g.max_pages = s.max_pages;
  g.num_pages = s.num_pages;
  g.slab = s.slab;
  g.scales = s.scales;
  g.row_bytes = lay.row_bytes;
  char* ws = static_cast<char*>(s.workspace);
  g.g_slab = reinterpret_cast<uint8_t*>(ws + lay.off_slab);
  g.g_scales = s.scales ? reinterpret_cast<uint16_t*>(ws + lay.off_scales) : nullptr;
  g.g_pt = reinterpret_cast<int32_t*>(ws + lay.off_pt);
  g.g_len = reinterpret_cast<int32_t*>(ws + lay.off_len);
  const dim3 grid((unsigned)((int64_t)batch * g.slices));
  if (lay.row_bytes == kDsmRow)
    sparse_gather_kernel<kDsmRow / 16><<<grid, kThreads, 0, stream>>>(g);
  else if (lay.row_bytes == kMlaDqk * 2)
    sparse_gather_kernel<kMlaDqk * 2 / 16><<<grid, kThreads, 0, stream>>>(g);
  else
    sparse_gather_kernel<kMlaDqk / 16><<<grid, kThreads, 0, stream>>>(g);
  return hipGetLastError();
}

}  // namespace kvq
