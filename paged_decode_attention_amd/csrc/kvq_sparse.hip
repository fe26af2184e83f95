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
// of exactly those rows.  One workgroup per sequence walks its list in chunks
// of 256 entries: an entry is taken when it is a position below the
// sequence's length on a page that is present; the taken ones of a chunk get
// consecutive places (a ballot count inside each wave, the wave totals
// through LDS), and the workgroup copies their code rows (16-byte moves) and
// scale rows into the workspace.  It then writes an identity page table for
// the compact sequence and its length.  The codes are moved, not decoded, so
// the decode sees exactly the stored rows.
#include "kvq_attn.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;

struct GatherArgs {
  const int32_t* topk;
  int64_t topk_stride;
  int k, kk;  // entries per list, and rows per compact sequence (k rounded up to a page)
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

__global__ __launch_bounds__(kThreads) void sparse_gather_kernel(GatherArgs g) {
  __shared__ int64_t s_src[kThreads];
  __shared__ int s_wave[kThreads / 64];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t L = g.seq_lens[b];
  const int64_t cap = (int64_t)g.max_pages * kPageSize;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int gpages = g.kk / kPageSize;
  int count = 0;  // rows placed so far (uniform)
  for (int i0 = 0; i0 < g.k; i0 += kThreads) {
    const int i = i0 + tid;
    const int64_t t = (i < g.k) ? g.topk[(int64_t)b * g.topk_stride + i] : -1;
    bool take = t >= 0 && t < L;
    int64_t page = -1;
    if (take) page = g.page_table[(int64_t)b * g.pt_stride + t / kPageSize];
    take = take && page >= 0 && page < g.num_pages;
    const uint64_t m = __builtin_amdgcn_ballot_w64(take);
    const int before = __builtin_popcountll(m & ((1ull << lane) - 1ull));
    if (lane == 0) s_wave[wave] = __builtin_popcountll(m);
    __syncthreads();
    int base = 0, chunk = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
      base += (w < wave) ? s_wave[w] : 0;
      chunk += s_wave[w];
    }
    if (take) s_src[base + before] = page * kPageSize + t % kPageSize;
    __syncthreads();
    // code rows, 16 bytes per thread per turn
    const int units = g.row_bytes / 16;
    for (int u = tid; u < chunk * units; u += kThreads) {
      const int r = u / units, c = u - r * units;
      const uint4 v = *reinterpret_cast<const uint4*>(g.slab + s_src[r] * g.row_bytes + c * 16);
      *reinterpret_cast<uint4*>(g.g_slab + ((int64_t)b * g.kk + count + r) * g.row_bytes + c * 16) = v;
    }
    if (g.scales) {
      for (int u = tid; u < chunk * (kNB / 2); u += kThreads) {  // two fp16 per turn
        const int r = u / (kNB / 2), c = u - r * (kNB / 2);
        const uint32_t v = *reinterpret_cast<const uint32_t*>(g.scales + s_src[r] * kNB + 2 * c);
        *reinterpret_cast<uint32_t*>(g.g_scales + ((int64_t)b * g.kk + count + r) * kNB + 2 * c) = v;
      }
    }
    count += chunk;
    __syncthreads();  // s_src and s_wave are reused by the next chunk
  }
  for (int p = tid; p < gpages; p += kThreads) g.g_pt[(int64_t)b * gpages + p] = b * gpages + p;
  if (tid == 0) g.g_len[b] = count;
}

}  // namespace

hipError_t launch_sparse_gather(const SparseArgs& s, const SparseLayout& lay, int batch,
                                hipStream_t stream) {
  GatherArgs g;
  g.topk = s.topk;
  g.topk_stride = s.topk_stride;
  g.k = s.k;
  g.kk = lay.kk;
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
  sparse_gather_kernel<<<batch, kThreads, 0, stream>>>(g);
  return hipGetLastError();
}

}  // namespace kvq
