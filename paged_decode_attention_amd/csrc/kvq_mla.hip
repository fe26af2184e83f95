// kvq_mla.hip -- paged decode attention over the shared MLA latent slab:
// one 576-element row per token serves as K (all 576) and V (the first 512),
// one KV head shared by up to 128 query heads (gfx950, bf16 MFMA).
//
// Sources: [PR113] "feat(kvcache): 8-bit DSV4 window/compressed KV behind
// --kv-cache-dtype" §What this adds (one 8-bit slab, one scale array beside
// it, K and V read from the same row), §Why the precision cost is small and
// §Testing (split-k decode); [PR25] "Experimental FP8 KV Cache" (the sparse
// MLA decode profile: 128 heads against one 576/512 latent row); [PR103]
// "feat(kvcache): 8-bit KV cache (q8_0 / fp8_e4m3) behind --kv-cache-dtype"
// §What (dequantize to bf16 before the dot, because the block scale runs
// along the reduction dimension).
//
// With every query head reading the same row, the work is a dense
// contraction: per 32-token tile, S = Q K^T is 128 x 32 x 576 and O += P V is
// 128 x 512 x 32.  The tile's codes are dequantized once (code * scale, one
// bf16 rounding, exactly kvq_dequant's rows) into LDS and then read by all
// four waves as MFMA operands:
//   - K rows, token-major [32][576 (+8 pad)], for S^T = K Q^T (16x16x32 bf16
//     MFMA: K as the A operand, Q^T from registers as B);
//   - V transposed, [512][32 (+pad)], for O^T = V^T P^T.  The tokens of a
//     tile sit in LDS in the order the S^T accumulator hands them to a lane,
//     so each lane's probabilities become its P^T operand without any
//     cross-lane movement.
// Wave w owns query heads 32w .. 32w+31 (two 16-head MFMA tiles); its O^T
// accumulator is 512 x 32 fp32 (256 registers per lane).  Tiles are double
// buffered: while tile j is multiplied, tile j+1's codes (already in
// registers) are dequantized into the other buffer and tile j+2's are loaded,
// with one block barrier per tile.
//
// Work item = (sequence, chunk of item_tokens tokens); items are enumerated
// on the device from seq_lens and a persistent grid strides over them.  A
// sequence that fits one item is written directly; otherwise each item
// stores its normalized output (bf16) and (m, l) for every head, and
// mla_merge_kernel combines them.
//
// Sparse top-k decode ([PR25] SPARSE_MLA_DECODE: K listed tokens per query;
// [PR113] §Testing: masked (-1) columns) is the same kernel with the list in
// place of the sequence: softmax attention over a set of rows does not depend
// on their order, so entry i of a list is token i of a sequence of K tokens,
// read from the slab row its position maps to through the page table, and an
// entry outside the sequence or on a missing page is a masked token.  Every
// list has K entries, so the items need no lengths from the device.
#include <type_traits>

#include "kvq_attn.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kW = 4;                 // waves per workgroup
constexpr int kT = 64 * kW;           // threads per workgroup
constexpr int kDqk = kMlaDqk;         // 576
constexpr int kDv = kMlaDv;           // 512
constexpr int kNB = kDqk / 32;        // scales per row (18)
constexpr int kTile = kMlaTile;       // tokens per LDS tile (two pages)
constexpr int kKS = kDqk + 8;         // bf16 per K row in LDS (1168 B: conflict-free reads)
constexpr int kVR = kTile + 8;        // bf16 per V^T row in LDS (80 B)
// V^T rows are padded by 8 more elements every 16 rows so that the 16-row
// stride of the writers falls on distinct banks.
constexpr int kVtElems = kDv * kVR + (kDv / 16) * 8;
// Output staging row (bf16): 512 + 8 keeps the 16-byte rows aligned.
constexpr int kStageRow = kDv + 8;
constexpr int kSlack = 64;            // log2-domain headroom above the softmax reference

__host__ __device__ constexpr int vt_index(int d, int pos) { return d * kVR + (d >> 4) * 8 + pos; }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// D = A B + C for a 16x32 A (lane l: row l%16, k = 8(l/16) .. +7), a 32x16 B
// (lane l: column l%16, the same k) and a 16x16 fp32 D (lane l: column l%16,
// rows 4(l/16) .. +3).
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// The same product for the score tiles, written so that its accumulator stays
// in ordinary VGPRs: the 512x32 fp32 P V accumulator of a wave fills all 256
// AGPRs, and the compiler would otherwise place these tiles there as well.
// The compiler treats the statement as opaque, so it does not pad the
// result's first VALU read; mfma16_v_settle() does that (more than the 18
// wait states an 8-pass XDL result needs before a VALU read).
__device__ __forceinline__ void mfma16_v_first(f32x4& d, u32x4 a, u32x4 b) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16_v(f32x4& d, u32x4 a, u32x4 b) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16_v_settle(f32x4& a, f32x4& b, f32x4& c, f32x4& d) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}

// ---- explicitly pipelined LDS operand reads ------------------------------------------
// The multiply phases read one 16-byte operand per lane per two MFMAs; to keep
// the matrix core busy, several reads must be in flight.  The reads are issued
// as ordered asm with immediate offsets, and each consumer waits with an
// explicit lgkmcnt: LDS operations complete in order, so "at most N
// outstanding" with N of this sequence's reads issued after the one needed
// guarantees it has landed (any other LDS or scalar operation in between only
// makes the wait stricter).
template <int OFF>
__device__ __forceinline__ void ds_read16(u32x4& d, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "i"(OFF));
}
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4& d) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(d) : "i"(N));
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)p;  // the low half of a flat LDS address is the LDS offset
}
template <int I, int N>
struct StaticFor {
  template <class F>
  __device__ __forceinline__ static void run(F&& f) {
    f(std::integral_constant<int, I>{});
    StaticFor<I + 1, N>::run(f);
  }
};
template <int N>
struct StaticFor<N, N> {
  template <class F>
  __device__ __forceinline__ static void run(F&&) {}
};
// The compiler does not count the asm LDS writes above, so it cannot be
// relied on to wait for them before a barrier: every barrier that publishes
// them is preceded by this.
__device__ __forceinline__ void lds_writes_done() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int OFF>
__device__ __forceinline__ void ds_write16(uint32_t addr, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(addr), "v"(v), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_write8(uint32_t addr, u32x2 v) {
  asm volatile("ds_write_b64 %0, %1 offset:%2" : : "v"(addr), "v"(v), "i"(OFF));
}
constexpr int cmin(int a, int b) { return a < b ? a : b; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int kAhead = 4;  // operand reads in flight
// The next tile's codes are loaded from inside the S^T multiplies, after
// read kLoadAt: any register reload the compiler places at the top of the
// tile then waits for its own load only, not for this tile's prefetch.
constexpr int kLoadAt = 3;
constexpr int kRing = kAhead + 1;
// Dequantization micro-steps of the next tile (one LDS write each), run from
// P V step kStoreAt on.
constexpr int kStoreSteps = 25;
constexpr int kStoreAt = 32 - kStoreSteps;
// LDS operations issued after P V read dt when step dt waits for it: the
// reads still ahead (at most kAhead - 1) and the writes of steps dt-4 .. dt-1.
constexpr int pv_wait(int dt) {
  int w = 0;
  for (int s = cmax(0, dt - kAhead); s < dt; ++s) w += (s >= kStoreAt) ? 1 : 0;
  return cmin(kAhead - 1, 31 - dt) + w;
}

struct MlaParams {
  DecodeArgs a;
  int item_tokens;   // a multiple of kTile
  float scale_log2;  // sm_scale * log2(e)
  int* prefix;       // [batch + 1] items before each sequence (written by block 0)
  float* part_ml;       // [items][n_q_heads][2]  (log2-domain reference, sum)
  uint16_t* part_out;   // [items][n_q_heads][512] bf16: the item's normalized output
};

template <int QT>
struct MlaGeo {
  static constexpr int ESZ = (QT == QT_BF16) ? 2 : 1;
  // code bytes per token row (the 656-byte row: its codes, scales and rope)
  static constexpr int ROWB = (QT == QT_DSM) ? kDsmRow : kDqk * ESZ;
  static constexpr int PAGEB = kPageSize * ROWB;    // code bytes per page
  static constexpr int SCLB = kPageSize * kNB * 2;  // scale bytes per page
  static constexpr int VW = 4 * ESZ;                // dwords of 16 V-part elements
  static constexpr int RW = (QT == QT_DSM) ? 4 : 2 * ESZ;  // dwords of 8 rope elements
};

// One thread's share of a tile's codes and scales, loaded a tile ahead.
//   V part: tokens 4*q4 .. 4*q4+3 of the tile, elements 16u .. 16u+15;
//   rope:   token rt of the tile, elements 512 + 8*p8 .. +7.
template <int QT>
struct MlaRaw {
  uint32_t v[4][MlaGeo<QT>::VW];
  uint32_t vs[4];
  uint32_t r[MlaGeo<QT>::RW];
  uint32_t rs;
  uint32_t okm;  // sparse lists: bit i for token 4*q4 + i, bit 4 for rope token rt (listed row present)
};

// The slab's code loads use the default cache policy: unlike the
// separate-K/V decode (whose streaming loads are non-temporal: 51 against
// 57 us over 8 x 16384 tokens, 16 q / 8 kv heads), this kernel ran faster
// with it (77.6 against 79.3 us per call at 163840 tokens; the 656-byte row
// unchanged).
constexpr int kSlabLoadPolicy = 0;

template <int N>
__device__ __forceinline__ void buf_load_dw(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t* o) {
  if constexpr (N == 8) {
    buf_load_dw<4>(rs, off, o);
    buf_load_dw<4>(rs, off + 16, o + 4);
  } else if constexpr (N == 4) {
    const u32x4 v = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kSlabLoadPolicy));
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  } else {
    static_assert(N == 2, "load width");
    const u32x2 v = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kSlabLoadPolicy));
    o[0] = v.x; o[1] = v.y;
  }
}

// Codes of one dword (four 8-bit codes, or two bf16) times the block scale,
// rounded once to bf16 pairs (the product is exact in fp32).
// (The 656-byte row's fp32 tile scales make the product inexact: it is
// rounded to fp32, then to bf16.)
template <int QT>
__device__ __forceinline__ void dequant_dword(uint32_t w, float s, uint32_t* o) {
  if constexpr (QT == QT_BF16) {
    o[0] = w;
  } else if constexpr (!qt_scaled(QT) && QT != QT_DSM) {  // cast codes: exact, no scale
    decode_dword_bf16x2<QT>(w, o);
  } else {
    float f[4];
    decode_dword<QT>(w, f);
    o[0] = pack_bf16x2(f[0] * s, f[1] * s);
    o[1] = pack_bf16x2(f[2] * s, f[3] * s);
  }
}

// A copy of x the compiler cannot see through (it recomputes what derives
// from it instead of holding that in registers).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ float scale_half(uint32_t w, int shift) {
  return f16_bits_to_f32((uint16_t)(w >> shift));
}

// Extend attention over the slab [PR103 §What: the quantized pool feeds the
// prefill / extend kernels; PR113 §Testing: prefill] runs the same kernel
// with the work numbered by new token: index v of the work list is new token
// i = v % M of sequence s = v / M (M = max_new); it attends to its
// sequence's first L_s - E_s + i + 1 positions (its causal end) through page
// row s, and reads / writes q and out row q_start[s] + i.  Indexes past a
// sequence's new tokens have no positions and no row.  Without q_start, v is
// the sequence itself.
__device__ __forceinline__ int mla_len(const DecodeArgs& a, int v) {
  if (!a.q_start) return clamped_len(a, v);
  const int s = v / a.max_new, i = v - s * a.max_new;
  const int E = a.q_start[s + 1] - a.q_start[s];
  return i < E ? max(clamped_len(a, s) - E + i + 1, 0) : 0;
}
__device__ __forceinline__ int mla_pt_row(const DecodeArgs& a, int v) {
  return a.q_start ? v / a.max_new : v;
}
__device__ __forceinline__ int64_t mla_row(const DecodeArgs& a, int v) {
  if (!a.q_start) return v;
  const int s = v / a.max_new, i = v - s * a.max_new;
  return i < a.q_start[s + 1] - a.q_start[s] ? (int64_t)a.q_start[s] + i : -1;
}

// Global loads of N dwords at a byte address (the sparse lists' rows, each
// at its own address); the default cache policy, as kSlabLoadPolicy.
template <int N>
__device__ __forceinline__ void glb_load_dw(const uint8_t* ptr, uint32_t* o) {
  if constexpr (N == 8) {
    glb_load_dw<4>(ptr, o);
    glb_load_dw<4>(ptr + 16, o + 4);
  } else if constexpr (N == 4) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(ptr);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  } else {
    static_assert(N == 2, "load width");
    const u32x2 v = *reinterpret_cast<const u32x2*>(ptr);
    o[0] = v.x; o[1] = v.y;
  }
}

// SP: a sparse list per sequence (a.topk).  The list's entries take the
// places of the sequence's positions: every sequence has topk_k of them, in
// ceil(topk_k / item_tokens) items; an entry's row in the slab is looked up
// once per item (the position through the page table, into s_rows), and an
// entry that is not taken is a masked token.
template <int QT, bool SP>
__global__ __launch_bounds__(kT) void mla_decode_kernel(MlaParams p) {
  using Gm = MlaGeo<QT>;
  constexpr int ESZ = Gm::ESZ, ROWB = Gm::ROWB, PAGEB = Gm::PAGEB, SCLB = Gm::SCLB;
  constexpr int VW = Gm::VW, RW = Gm::RW;
  constexpr int EPD = (QT == QT_BF16) ? 1 : 2;  // bf16 pairs per code dword
  constexpr int RPD = (QT == QT_BF16 || QT == QT_DSM) ? 1 : 2;  // ... per rope dword
  // two tile buffers (K rows, V^T); at the end of an item the same memory
  // stages each wave's output rows
  __shared__ __attribute__((aligned(16))) uint16_t s_tiles[2 * kTile * kKS + 2 * kVtElems];
  auto kbuf = [&](int buf) { return s_tiles + buf * (kTile * kKS); };
  auto vbuf = [&](int buf) { return s_tiles + 2 * kTile * kKS + buf * kVtElems; };
  __shared__ int s_wave[kW];
  __shared__ int s_flag[3];  // per-tile restart votes, rotating
  extern __shared__ int s_prefix[];  // [batch + 1] (SP: unused)
  // SP: slab row of each of the item's entries (-1: not taken)
  __shared__ int s_rows[SP ? kMlaMaxItemPages * kPageSize : 1];

  const DecodeArgs& a = p.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g = lane >> 4;
  const int Hq = a.n_q_heads;

  // SP: every list has the same number of entries, so the same item count
  const int sp_items = SP ? (a.topk_k + p.item_tokens - 1) / p.item_tokens : 0;
  int total;
  if constexpr (SP) {
    total = a.batch * sp_items;
    if (blockIdx.x == 0)
      for (int b = tid; b <= a.batch; b += kT) p.prefix[b] = b * sp_items;
  } else {
    build_prefix_with<kT>(a, p.item_tokens, 1, s_prefix, s_wave,
                          [&](int v) { return mla_len(a, v); });
    total = s_prefix[a.batch];
    if (blockIdx.x == 0)
      for (int b = tid; b <= a.batch; b += kT) p.prefix[b] = s_prefix[b];
    // a sequence with no valid length has no items: its output is 0, lse -inf
    for (int b = blockIdx.x; b < a.batch; b += gridDim.x) {
      if (s_prefix[b] != s_prefix[b + 1]) continue;
      const int64_t row = mla_row(a, b);
      if (row < 0) continue;  // no such new token
      for (int i = tid; i < Hq * kDv; i += kT) a.out[row * Hq * kDv + i] = 0;
      if (a.lse)
        for (int h = tid; h < Hq; h += kT) a.lse[row * Hq + h] = -INFINITY;
    }
  }

  // ---- tile geometry ----------------------------------------------------------------
  // Tile token t (0..31, natural order; t < 16 on the tile's first page) is
  // K row rho(t) = 16*((t>>2)&1) + 4*(t>>3) + (t&3) in LDS, so that MFMA row
  // tile tt, row n of the S^T product is token 8*(n>>2) + 4*tt + (n&3).  A
  // lane in group g then holds tokens 8g .. 8g+7 of the tile after the
  // softmax, which is exactly its k-slot range of the P^T operand, and V^T
  // keeps tokens in natural order.
  //
  // Loaders: lane l of wave w owns token quad q = 2w + ((l>>3)&1) (tokens
  // 4q .. 4q+3, all on page w>>1) and the 16-element unit u = (l&7) |
  // ((l>>4)<<3) of the latent part; and rope token rt = 8w + (l>>3), 8-element
  // unit p8 = l&7.  With this assignment each group of 8 (16-byte writes) or
  // 16 lanes (8-byte writes) covers all LDS banks once: K rows are written
  // in 16-byte halves, lanes with (u>>2)&1 set writing their second half
  // first.  The offsets are recomputed from an opaque copy of tid where they
  // are used, so they do not stay live across the multiply phase.
  const int wpage = wave >> 1;

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    // ---- describe the item (uniform over the block) ------------------------------
    int b, chunk;
    if constexpr (SP) {
      b = item / sp_items;
      chunk = item - b * sp_items;
    } else {
      int lo = 0, hi = a.batch - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_prefix[mid] <= item) lo = mid; else hi = mid - 1;
      }
      b = lo;
      chunk = item - s_prefix[b];
    }
    const int L = SP ? a.topk_k : mla_len(a, b);
    const int64_t orow = mla_row(a, b);  // valid: b has work
    const int nc = (L + p.item_tokens - 1) / p.item_tokens;
    const int t0 = chunk * p.item_tokens;
    const int nt = min(p.item_tokens, L - t0);
    const int ntiles = (nt + kTile - 1) / kTile;
    const int npages = (nt + kPageSize - 1) / kPageSize;

    // page ids of the item: lane k holds page column t0/16 + k; masked -> -1
    int pid = -1;
    if (!SP && lane < npages) {
      const int v = a.page_table[(int64_t)mla_pt_row(a, b) * a.pt_stride + t0 / kPageSize + lane];
      pid = (v >= 0 && (int64_t)v < a.num_pages) ? v : -1;
    }
    // page id of tile j's page k (k = 0, 1); -1 past the item
    auto page_of = [&](int j, int k) {
      const int c = 2 * j + k;
      return c < 64 ? __builtin_amdgcn_readlane(pid, c) : -1;
    };

    // this wave's 32 query heads as MFMA B operands: qr[ht][ks] holds, for
    // head 32w + 16ht + (l%16), elements 32ks + 8(l/16) .. +7 (loaded below,
    // after the first tile's codes)
    u32x4 qr[2][kNB];

    if constexpr (SP) {
      // the slab row of each entry of the item: taken when 0 <= position <
      // the sequence's length and its page is present (the earlier readers
      // of s_rows are past the previous item's last tile barrier)
      const int Ls = clamped_len(a, b);
      for (int e = tid; e < nt; e += kT) {
        const int pos = a.topk[(int64_t)b * a.topk_stride + t0 + e];
        int row = -1;
        if (pos >= 0 && pos < Ls) {
          const int pg = a.page_table[(int64_t)b * a.pt_stride + pos / kPageSize];
          if (pg >= 0 && (int64_t)pg < a.num_pages) row = pg * kPageSize + pos % kPageSize;
        }
        s_rows[e] = row;
      }
      __syncthreads();
    }

    auto load_tile = [&](int j, MlaRaw<QT>& R) {
      const int t = opaque(tid);
      const int l = t & 63, q = 2 * (t >> 6) + ((l >> 3) & 1), u = (l & 7) | ((l >> 4) << 3);
      const int rt = t >> 3, p8 = t & 7;
      const uint32_t vbase = (uint32_t)((4 * (q & 3)) * ROWB + u * 16 * ESZ);
      const uint32_t sbase = (uint32_t)((4 * (q & 3)) * kNB * 2 + (u >> 2) * 4);
      const uint32_t roff = (uint32_t)((rt & (kPageSize - 1)) * ROWB +
                                       (QT == QT_DSM ? kDsmLatent + 16 + 16 * p8 : (kDv + 8 * p8) * ESZ));
      const uint32_t rsoff = (uint32_t)((rt & (kPageSize - 1)) * kNB * 2 + (kDv / 32) * 2);
      if constexpr (SP) {
        // each token at its own row (row 0 stands in for an entry not taken)
        const int base = kTile * j;
        int rr[4];
        uint32_t okm = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = base + 4 * q + i;
          const int r = e < nt ? s_rows[e] : -1;
          okm |= (r >= 0 ? 1u : 0u) << i;
          rr[i] = max(r, 0);
        }
        const int er = base + rt;
        const int rrow = er < nt ? s_rows[er] : -1;
        okm |= (rrow >= 0 ? 1u : 0u) << 4;
        const int64_t rb = (int64_t)max(rrow, 0);
        R.okm = okm;
        const uint8_t* slab = a.k_pool;
#pragma unroll
        for (int i = 0; i < 4; ++i) glb_load_dw<VW>(slab + (int64_t)rr[i] * ROWB + u * 16 * ESZ, R.v[i]);
        glb_load_dw<RW>(slab + rb * ROWB + (roff - (uint32_t)((rt & (kPageSize - 1)) * ROWB)), R.r);
        if constexpr (QT == QT_DSM) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            R.vs[i] = *reinterpret_cast<const uint32_t*>(slab + (int64_t)rr[i] * ROWB + kDsmLatent + 4 * (u >> 3));
        }
        if constexpr (qt_scaled(QT)) {
          const uint8_t* sc = reinterpret_cast<const uint8_t*>(a.k_scales);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            R.vs[i] = *reinterpret_cast<const uint32_t*>(sc + (int64_t)rr[i] * (kNB * 2) + (u >> 2) * 4);
          R.rs = *reinterpret_cast<const uint32_t*>(sc + rb * (kNB * 2) + (kDv / 32) * 2);
        }
        return;
      }
      const int P = max(__builtin_amdgcn_readfirstlane(page_of(j, wpage)), 0);
      const auto rc = page_rsrc(a.k_pool + (int64_t)P * PAGEB, PAGEB);
#pragma unroll
      for (int i = 0; i < 4; ++i) buf_load_dw<VW>(rc, vbase + i * ROWB, R.v[i]);
      buf_load_dw<RW>(rc, roff, R.r);
      if constexpr (QT == QT_DSM) {  // the fp32 scale of unit u's 128-element tile, per token
#pragma unroll
        for (int i = 0; i < 4; ++i)
          R.vs[i] = __builtin_amdgcn_raw_buffer_load_b32(
              rc, (uint32_t)((4 * (q & 3) + i) * ROWB + kDsmLatent + 4 * (u >> 3)), 0, 0);
      }
      if constexpr (qt_scaled(QT)) {
        const auto rs = page_rsrc(a.k_scales + (int64_t)P * (SCLB / 2), SCLB);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          R.vs[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, sbase + i * kNB * 2, 0, 0);
        R.rs = __builtin_amdgcn_raw_buffer_load_b32(rs, rsoff, 0, 0);
      }
    };

    // Dequantizing tile j from registers into LDS buffer `buf`, as 25
    // micro-steps of one LDS write each (so they can be spread between the
    // multiplies of the tile being computed):
    //   0..3   first half of the unit, token i: dequantize, write its K row part
    //   4..11  first half, element e: write V^T row 16u + 8h + e (4 tokens)
    //   12..23 the same for the second half
    //   24     rope part of token rt
    // Rows of masked pages or past the item end are written as zeros.
    struct StoreState {
      uint32_t kb, vb, rb;  // LDS byte addresses: K row part, V^T element 0, rope
      int h0;               // the half written first
      float sv[4];
      bool ok[4], okr;
      uint32_t hv[4][4];    // the current half: 4 tokens x 4 bf16 pairs
    } st;
    auto store_begin = [&](int j, const MlaRaw<QT>& R, int buf) {
      const int t = opaque(tid);
      const int l = t & 63, q = 2 * (t >> 6) + ((l >> 3) & 1), u = (l & 7) | ((l >> 4) << 3);
      const int rt = t >> 3, p8 = t & 7;
      const int row_q = 16 * (q & 1) + 4 * (q >> 1);
      const int row_r = 16 * ((rt >> 2) & 1) + 4 * (rt >> 3) + (rt & 3);
      st.kb = lds_addr(kbuf(buf)) + (uint32_t)(row_q * kKS * 2 + 32 * u);
      st.vb = lds_addr(vbuf(buf)) + (uint32_t)(vt_index(16 * u, 4 * q) * 2);
      st.rb = lds_addr(kbuf(buf)) + (uint32_t)(row_r * kKS * 2 + (kDv + 8 * p8) * 2);
      st.h0 = (u >> 2) & 1;
      const bool page_ok = SP || page_of(j, wpage) >= 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        st.ok[i] = page_ok && (kTile * j + 4 * q + i < nt) && (!SP || ((R.okm >> i) & 1u));
        st.sv[i] = (QT == QT_DSM) ? __uint_as_float(R.vs[i])
                   : qt_scaled(QT) ? scale_half(R.vs[i], ((u >> 1) & 1) * 16) : 1.0f;
      }
      st.okr = page_ok && (kTile * j + rt < nt) && (!SP || ((R.okm >> 4) & 1u));
    };
    auto store_step = [&](auto sc, const MlaRaw<QT>& R) {
      constexpr int S = decltype(sc)::value;
      if constexpr (S < 24 && S % 12 < 4) {  // token i of half hh: dequantize
        constexpr int hh = S / 12, i = S % 12;
        const int h = st.h0 ^ hh;  // lane-dependent half
        uint32_t c[VW / 2];
#pragma unroll
        for (int k = 0; k < VW / 2; ++k) c[k] = h ? R.v[i][VW / 2 + k] : R.v[i][k];
        uint32_t* o = st.hv[i];
        if constexpr (QT == QT_BF16) {
#pragma unroll
          for (int k = 0; k < 4; ++k) o[k] = c[k];
        } else {
          dequant_dword<QT>(c[0], st.sv[i], o);
          dequant_dword<QT>(c[1], st.sv[i], o + 2);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = st.ok[i] ? o[k] : 0u;
        ds_write16<i * kKS * 2>(st.kb + 16 * h, u32x4{o[0], o[1], o[2], o[3]});
      } else if constexpr (S < 24) {  // element e of half hh: V^T row, 4 tokens
        constexpr int hh = S / 12, e = S % 12 - 4;
        const int h = st.h0 ^ hh;
        constexpr uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t w01 = __builtin_amdgcn_perm(st.hv[1][e >> 1], st.hv[0][e >> 1], sel);
        const uint32_t w23 = __builtin_amdgcn_perm(st.hv[3][e >> 1], st.hv[2][e >> 1], sel);
        ds_write8<e * kVR * 2>(st.vb + (uint32_t)(h * 8 * kVR * 2), u32x2{w01, w23});
      } else {  // rope
        const int t = opaque(tid);
        const float s = qt_scaled(QT) ? scale_half(R.rs, ((t & 7) >> 2) * 16) : 1.0f;
        uint32_t rw[4];
#pragma unroll
        for (int k = 0; k < RW; ++k) {
          if constexpr (QT == QT_DSM)
            rw[k] = R.r[k];  // the rope is stored as bf16
          else
            dequant_dword<QT>(R.r[k], s, &rw[k * RPD]);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) rw[k] = st.okr ? rw[k] : 0u;
        ds_write16<0>(st.rb, u32x4{rw[0], rw[1], rw[2], rw[3]});
      }
    };

    // Softmax reference per head (lane column): fixed for a pass over the
    // item.  It is taken from the first tile with a valid score; a score more
    // than kSlack above it ends the pass, and the item is run again from its
    // first tile with the larger reference.  The accumulators are thus never
    // rescaled, only cleared (exact: 2^(s - ref) <= 2^kSlack keeps every sum
    // far inside fp32 range).
    float mref[2] = {-INFINITY, -INFINITY}, mseen[2] = {-INFINITY, -INFINITY};
    float lsum[2];
    f32x4 acc[kDv / 16][2];

    // Tile j from LDS buffer `buf`; meanwhile tile j+1 (in R) is dequantized
    // into the other buffer, and then tile j+2 is loaded into R.
    auto compute = [&](int j, int buf, int fslot, MlaRaw<QT>& R) {
      // S^T = K Q^T.  Read r = 2ks + tt is K rows 16tt + l%16 (see rho),
      // elements 32ks + 8g .. +7.
      f32x4 S[2][2];
      {
        constexpr int NR = 2 * kNB;
        const uint32_t ka = lds_addr(kbuf(buf) + n16 * kKS + 8 * g);
        u32x4 ring[kRing];
        StaticFor<0, kAhead>::run([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          ds_read16<(r % 2) * 16 * kKS * 2 + (r / 2) * 64>(ring[r], ka);
        });
        StaticFor<0, NR>::run([&](auto rc) {
          constexpr int r = decltype(rc)::value, ks = r / 2, tt = r % 2;
          lgkm_wait<cmin(kAhead - 1, NR - 1 - r)>(ring[r % kRing]);
          if constexpr (ks == 0) {
            mfma16_v_first(S[tt][0], ring[r % kRing], qr[0][ks]);
            mfma16_v_first(S[tt][1], ring[r % kRing], qr[1][ks]);
          } else {
            mfma16_v(S[tt][0], ring[r % kRing], qr[0][ks]);
            mfma16_v(S[tt][1], ring[r % kRing], qr[1][ks]);
          }
          if constexpr (r + kAhead < NR) {
            constexpr int n = r + kAhead;
            ds_read16<(n % 2) * 16 * kKS * 2 + (n / 2) * 64>(ring[n % kRing], ka);
          }
          // tile j+1's codes (dequantized during the P V multiplies below)
          if constexpr (r == kLoadAt)
            if (j + 1 < ntiles && j > 0) load_tile(j + 1, R);
        });
      }
      mfma16_v_settle(S[0][0], S[0][1], S[1][0], S[1][1]);
      // lane group g holds tokens 8g + 4tt + r: page 0 for g < 2
      bool pok;
      uint64_t tmask = 0;  // SP: the tile's listed rows present
      if constexpr (SP) {
        const int e = kTile * j + lane;
        tmask = __builtin_amdgcn_ballot_w64(lane < kTile && e < nt && s_rows[e] >= 0);
        pok = true;
      } else {
        const bool ok0 = page_of(j, 0) >= 0, ok1 = page_of(j, 1) >= 0;
        pok = (g < 2) ? ok0 : ok1;
      }
      u32x4 pk[2];
      bool over = false;
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        float sc[8], t = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tok = kTile * j + 8 * g + 4 * tt + r;
            const bool ok = SP ? ((tmask >> (8 * g + 4 * tt + r)) & 1u) != 0 : (pok && tok < nt);
            const float v = ok ? S[tt][ht][r] * p.scale_log2 : -INFINITY;
            sc[4 * tt + r] = v;
            t = fmaxf(t, v);
          }
        t = max_xor32(max_xor16(t));  // the tile max of this head
        mseen[ht] = fmaxf(mseen[ht], t);
        if (mref[ht] == -INFINITY) mref[ht] = t;  // nothing accumulated yet
        over |= t > mref[ht] + (float)kSlack;
        float pr[8], ls = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          pr[i] = exp2_rel(sc[i], mref[ht]);
          ls += pr[i];
        }
        lsum[ht] += ls;
        pk[ht] = u32x4{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                       pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
      }
      if (over) s_flag[fslot] = 1;
      // O^T += V^T P^T; read dt is V^T rows 16dt + l%16, tokens 8g .. 8g+7.
      // From step kStoreAt on, each step also runs one micro-step of tile
      // j+1's dequantization (one LDS write more per step, counted in the
      // waits).
      store_begin(j + 1, R, buf ^ 1);
      {
        constexpr int NR = kDv / 16;
        constexpr int STEP = vt_index(16, 0) * 2;  // bytes between 16-row groups
        const uint32_t va = lds_addr(vbuf(buf) + vt_index(n16, 8 * g));
        u32x4 ring[kRing];
        StaticFor<0, kAhead>::run([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          ds_read16<r * STEP>(ring[r], va);
        });
        StaticFor<0, NR>::run([&](auto rc) {
          constexpr int dt = decltype(rc)::value;
          lgkm_wait<pv_wait(dt)>(ring[dt % kRing]);
          acc[dt][0] = mfma16(ring[dt % kRing], pk[0], acc[dt][0]);
          acc[dt][1] = mfma16(ring[dt % kRing], pk[1], acc[dt][1]);
          if constexpr (dt + kAhead < NR) ds_read16<(dt + kAhead) * STEP>(ring[(dt + kAhead) % kRing], va);
          if constexpr (dt >= kStoreAt) store_step(std::integral_constant<int, dt - kStoreAt>{}, R);
        });
      }
    };

    // The first tile's codes are requested before the query: the query (147
    // KB per workgroup) takes the longest to arrive, and the first tile is
    // dequantized while it does.
    MlaRaw<QT> R;
    load_tile(0, R);
    {
      // coalesced: lane L reads 16 bytes of head L / 4 (piece L % 4 of each
      // 64-byte k span); the fragment lane L needs is held by lane
      // 4 (L % 16) + L / 16
      const int src_lane = 4 * n16 + g;
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const int hl = 32 * wave + 16 * ht + (lane >> 2);
        const uint16_t* qrow = a.q + (orow * Hq + (hl < Hq ? hl : 0)) * kDqk + 8 * (lane & 3);
#pragma unroll
        for (int ks = 0; ks < kNB; ++ks) qr[ht][ks] = *reinterpret_cast<const u32x4*>(qrow + 32 * ks);
      }
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const bool dead = 32 * wave + 16 * ht + n16 >= Hq;
#pragma unroll
        for (int ks = 0; ks < kNB; ++ks) {
          u32x4 v;
#pragma unroll
          for (int c = 0; c < 4; ++c) v[c] = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * src_lane, (int)qr[ht][ks][c]);
          if (dead) v = u32x4{0, 0, 0, 0};
          qr[ht][ks] = v;
        }
      }
    }
    bool again = false;
    while (true) {  // passes over the item (a second one only after a restart)
#pragma unroll
      for (int dt = 0; dt < kDv / 16; ++dt) {
        acc[dt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc[dt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      lsum[0] = lsum[1] = 0.0f;
      if (again) load_tile(0, R);
      again = true;
      __syncthreads();  // earlier reads of both buffers and of the votes are done
      if (tid < 3) s_flag[tid] = 0;
      store_begin(0, R, 0);
      StaticFor<0, kStoreSteps>::run([&](auto sc) { store_step(sc, R); });
      if (ntiles > 1) load_tile(1, R);
      lds_writes_done();
      __syncthreads();
      // Tile j votes into slot j % 3 and is decided after its barrier.  The
      // slot of tile j+1 is cleared before that barrier: its last readers
      // (tile j-2's decision) are past barrier j-1, its writers after j.
      // (The last tile also writes its spare buffer, with zeros: harmless,
      // that buffer is not read before the next barrier.)
      bool restart = false;
      for (int j = 0, slot = 0; j < ntiles; ++j) {
        const int next = (slot == 2) ? 0 : slot + 1;
        compute(j, j & 1, slot, R);
        if (tid == 0) s_flag[next] = 0;
        lds_writes_done();
        __syncthreads();
        restart = s_flag[slot] != 0;  // the same for every thread
        if (restart) break;
        slot = next;
      }
      if (!restart) break;
      mref[0] = mseen[0];
      mref[1] = mseen[1];
    }

    // ---- item result --------------------------------------------------------------
    // Each head's row, normalized and rounded to bf16, goes to the output (a
    // sequence that fits one item) or to the item's partial slot.  The rows
    // are staged in LDS (the tile buffers are free after the loop's last
    // barrier) so that every global store writes 1 KB contiguous per wave.
    {
      // Lane-dependent offsets are recomputed here from an opaque copy of
      // tid: values kept from the prologue end up spilled, and each reload is
      // a memory round trip that also waits for every earlier store.
      const int t = opaque(tid);
      const int l = t & 63, nn = l & 15, gg = l >> 4;
      uint16_t* stage = s_tiles + wave * (32 * kStageRow);
      float Lh[2];
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const float Ls = sum_xor32(sum_xor16(lsum[ht]));
        Lh[ht] = Ls;
        const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
        uint16_t* srow = stage + (16 * ht + nn) * kStageRow + 4 * gg;
#pragma unroll
        for (int dt = 0; dt < kDv / 16; ++dt) {
          const f32x4 v = acc[dt][ht];
          *reinterpret_cast<u32x2*>(srow + 16 * dt) =
              u32x2{pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv)};
        }
      }
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const int h = 32 * wave + 16 * ht + nn;
        if (gg == 0 && h < Hq) {
          if (nc == 1) {
            if (a.lse)
              a.lse[orow * Hq + h] =
                  (mref[ht] == -INFINITY) ? -INFINITY : (mref[ht] + log2f(Lh[ht])) * kLn2;
          } else {
            *reinterpret_cast<float2*>(p.part_ml + ((int64_t)item * Hq + h) * 2) =
                make_float2(mref[ht], Lh[ht]);
          }
        }
      }
      __builtin_amdgcn_wave_barrier();  // the stage is private to the wave
      // The wave's 32 rows: every LDS read first, then the global stores as
      // buffer stores through a descriptor that covers only the wave's heads
      // below Hq (stores past it are dropped), so no store waits on another.
      const int rows = __builtin_amdgcn_readfirstlane(min(32, max(Hq - 32 * wave, 0)));
      const uint64_t da = reinterpret_cast<uint64_t>(
          ((nc == 1) ? a.out + orow * Hq * kDv : p.part_out + (int64_t)item * Hq * kDv) +
          (int64_t)32 * wave * kDv);
      const uint64_t dsa = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(da >> 32)) << 32) |
                           (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)da);
      const auto rd = page_rsrc(reinterpret_cast<const void*>(dsa), rows * kDv * 2);
      const uint16_t* src = stage + 8 * l;
      u32x4 o[32];
#pragma unroll
      for (int r = 0; r < 32; ++r) o[r] = *reinterpret_cast<const u32x4*>(src + r * kStageRow);
#pragma unroll
      for (int r = 0; r < 32; ++r)
        __builtin_amdgcn_raw_buffer_store_b128(o[r], rd, r * kDv * 2 + 16 * l, 0, 0);
    }
  }
}

// ---- split-K merge -------------------------------------------------------------------
// Block = (sequence b, head h, half of the columns); 16 groups of 32 threads
// take every 16th chunk, a thread 8 columns.  The first kAheadRows chunk rows
// of every thread are requested before anything else, the chunks' (m, l)
// beside them (wave 0, all of a lane's chunks at once); the weights are
// formed while those rows arrive.
// With w_c = 2^(m_c - M) l_c: O = sum_c w_c O_c / sum_c w_c (O_c the chunk's
// normalized output) and lse = M + log2(sum_c w_c) in log2 units.
constexpr int kMergeGroups = 16;
constexpr int kMergeCols = kDv / 2;
constexpr int kMergeThreads = kMergeGroups * (kMergeCols / 8);
constexpr int kAheadRows = 8;                          // chunk rows per thread in flight
constexpr int kMlPerLane = kMlaMaxChunks / 64;         // (m, l) pairs per lane of wave 0

__global__ __launch_bounds__(kMergeThreads) void mla_merge_kernel(MlaParams p) {
  const DecodeArgs& a = p.a;
  const int Hq = a.n_q_heads;
  const int half = blockIdx.x & 1, bh = blockIdx.x >> 1;
  const int h = bh % Hq, b = bh / Hq;
  const int first = p.prefix[b];
  const int nc = p.prefix[b + 1] - first;
  if (nc <= 1) return;  // written by the decode kernel itself
  __shared__ float s_w[kMlaMaxChunks];
  __shared__ __attribute__((aligned(16))) float s_red[kMergeGroups][kMergeCols];
  __shared__ float s_L;
  const int tid = threadIdx.x, lane = tid & 63;
  const int grp = tid >> 5, j = tid & 31;
  const int d0 = half * kMergeCols + 8 * j;
  const uint16_t* src = p.part_out + ((int64_t)first * Hq + h) * kDv + d0;
  const int64_t cstride = (int64_t)Hq * kDv;
  // the first rows of this thread's chunks, requested at once
  u32x4 x0[kAheadRows];
#pragma unroll
  for (int k = 0; k < kAheadRows; ++k) {
    const int c = grp + k * kMergeGroups;
    x0[k] = c < nc ? *reinterpret_cast<const u32x4*>(src + (int64_t)c * cstride) : u32x4{0, 0, 0, 0};
  }
  if (tid < 64) {
    float2 ml[kMlPerLane];
#pragma unroll
    for (int k = 0; k < kMlPerLane; ++k) {
      const int c = lane + 64 * k;
      ml[k] = c < nc ? *reinterpret_cast<const float2*>(p.part_ml + ((int64_t)(first + c) * Hq + h) * 2)
                     : make_float2(-INFINITY, 0.0f);
    }
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kMlPerLane; ++k) M = fmaxf(M, ml[k].x);
    M = stride_max<1>(M);
    float Ls = 0.0f;
#pragma unroll
    for (int k = 0; k < kMlPerLane; ++k) {
      const int c = lane + 64 * k;
      if (c < nc) {
        const float w = exp2_rel(ml[k].x, M) * ml[k].y;
        s_w[c] = w;
        Ls += w;
      }
    }
    Ls = stride_sum<1>(Ls);
    if (lane == 0) {
      s_L = Ls;
      if (a.lse && half == 0)
        a.lse[mla_row(a, b) * Hq + h] = (Ls > 0.0f) ? (M + log2f(Ls)) * kLn2 : -INFINITY;
    }
  }
  __syncthreads();
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](const u32x4& x, float w) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] += w * bf16_lo(x[k]);
      v[2 * k + 1] += w * bf16_hi(x[k]);
    }
  };
#pragma unroll
  for (int k = 0; k < kAheadRows; ++k) {
    const int c = grp + k * kMergeGroups;
    if (c < nc) add(x0[k], s_w[c]);
  }
  int c = grp + kAheadRows * kMergeGroups;
  for (; c + 3 * kMergeGroups < nc; c += 4 * kMergeGroups) {
    u32x4 x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      x[k] = *reinterpret_cast<const u32x4*>(src + (int64_t)(c + k * kMergeGroups) * cstride);
#pragma unroll
    for (int k = 0; k < 4; ++k) add(x[k], s_w[c + k * kMergeGroups]);
  }
  for (; c < nc; c += kMergeGroups) add(*reinterpret_cast<const u32x4*>(src + (int64_t)c * cstride), s_w[c]);
#pragma unroll
  for (int k = 0; k < 8; ++k) s_red[grp][8 * j + k] = v[k];
  __syncthreads();
  if (tid < kMergeCols) {
    float t = 0.0f;
#pragma unroll
    for (int k = 0; k < kMergeGroups; ++k) t += s_red[k][tid];
    const float Ls = s_L;
    a.out[(mla_row(a, b) * Hq + h) * kDv + half * kMergeCols + tid] =
        (uint16_t)bf16_rne(Ls > 0.0f ? t / Ls : 0.0f);
  }
}

template <int QT>
hipError_t launch_q(const MlaParams& mp, int grid, int merge_grid, hipStream_t s) {
  if (mp.a.topk) {
    mla_decode_kernel<QT, true><<<grid, kT, 0, s>>>(mp);
  } else {
    const size_t dyn = (size_t)(mp.a.batch + 1) * sizeof(int);
    mla_decode_kernel<QT, false><<<grid, kT, dyn, s>>>(mp);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || merge_grid == 0) return e;
  mla_merge_kernel<<<merge_grid, kMergeThreads, 0, s>>>(mp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mla_decode(const DecodeArgs& a, const DecodePlan& plan, int num_cus,
                             hipStream_t s) {
  char* ws = static_cast<char*>(a.workspace);
  MlaParams mp;
  mp.a = a;
  mp.item_tokens = plan.item_pages * kPageSize;
  mp.scale_log2 = a.sm_scale * kLog2e;
  mp.prefix = reinterpret_cast<int*>(ws + plan.off_prefix);
  mp.part_ml = reinterpret_cast<float*>(ws + plan.off_ml);
  mp.part_out = reinterpret_cast<uint16_t*>(ws + plan.off_acc);
  int64_t grid = num_cus;  // one workgroup per CU fits the tiles' LDS
  if (grid > plan.max_items) grid = plan.max_items;
  if (a.items_hint > 0 && grid > a.items_hint) grid = a.items_hint;  // exact from host lengths
  if (grid < 1) grid = 1;
  const int64_t max_chunks = a.topk ? (a.topk_k + mp.item_tokens - 1) / mp.item_tokens
                                    : (a.max_pages + plan.item_pages - 1) / plan.item_pages;
  const int merge_grid = (max_chunks > 1) ? a.batch * a.n_q_heads * 2 : 0;
  switch (a.qtype) {
    case QT_BF16: return launch_q<QT_BF16>(mp, (int)grid, merge_grid, s);
    case QT_FP8: return launch_q<QT_FP8>(mp, (int)grid, merge_grid, s);
    case QT_FP8C: return launch_q<QT_FP8C>(mp, (int)grid, merge_grid, s);
    case QT_BF8C: return launch_q<QT_BF8C>(mp, (int)grid, merge_grid, s);
    case QT_DSM: return launch_q<QT_DSM>(mp, (int)grid, merge_grid, s);
    default: return launch_q<QT_Q8>(mp, (int)grid, merge_grid, s);
  }
}

}  // namespace kvq
