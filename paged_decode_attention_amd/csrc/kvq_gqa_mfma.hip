// kvq_gqa_mfma.hip -- paged decode attention over separate K/V pools for
// wide query groups (8 to 16 query heads per kv head) on the matrix cores
// (gfx950, bf16 MFMA, no LDS in the streaming loop).
//
// Sources: [PR103] "feat(kvcache): 8-bit KV cache (q8_0 / fp8_e4m3) behind
// --kv-cache-dtype" §What (dequantize before the dot, because the block scale
// runs along head_dim); [PR113] "feat(kvcache): 8-bit DSV4 window/compressed
// KV behind --kv-cache-dtype" §Testing (split-k decode, masked (-1) columns).
//
// With G query heads sharing a kv head, every K and V element feeds G dot
// products; at G >= 8 the VALU formulation runs out of issue slots before
// HBM is busy, so the products move to the matrix cores.  The G heads of a
// kv head (padded to 16) form the N dimension of every MFMA; tokens and
// head_dim elements come straight from registers:
//   - S^T = K Q^T per page (16 tokens) with v_mfma_f32_16x16x32_bf16: lane
//     (row n, group g) holds 8 codes of token n, elements 32ks + 8g .. +7, so
//     each k-step is exactly one 32-element scale block.  8-bit codes are
//     exact in bf16; every block has its own product tile, and the block
//     scales (per token, per block) weight the tiles in fp32:
//     s_t = sum_ks scale[t][ks] * (code_t . q)_ks.
//   - O^T += V^T P^T per page with v_mfma_f32_16x16x16_bf16: the S^T tile
//     hands lane (head n, group g) the probabilities of tokens 4g .. 4g+3,
//     which is its P^T operand as is.  V^T needs lane (row n, group g) to
//     hold V[4g .. 4g+3][dv]: the lane loads D/16 consecutive codes of each
//     of those 4 tokens (dv = (D/16)n .. +D/16) and transposes them in
//     registers (byte permutes), so tile i's row n is dv = (D/16)n + i.  The
//     V scale of (token, block) is the same for all of a lane's dv, so V is
//     dequantized on the way (one multiply per element).
// Each of the four waves streams its own pages with the next page's loads in
// flight; the waves are merged through LDS at the end of a work item, and
// split-K items are merged by the last workgroup of their (sequence, kv
// head, head group), as in the VALU kernel.
//
// The same kernel runs causal extend (prefill) attention [PR103 §What: the
// quantized pool feeds the prefill / extend kernels as well; PR113 §Testing:
// prefill]: a kv head's query rows are then its sequence's new tokens x G
// heads (token-major), 16 of them per column tile, each column with its own
// causal end; up to head_dim 128 a work item carries two tiles, computed by
// every wave over the same pages.
#include "kvq_attn.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kW = kDecodeWaves;
constexpr int kT = 64 * kW;
constexpr int kN = 16;  // query rows (heads, or new tokens x heads) per MFMA column tile
constexpr int kSharedTileGroups = 4;  // see launch_d

// Lane j of each row of 16 lanes, to every lane of the row (DPP row_newbcast).
// j is a constant once the callers' loops are unrolled; the switch folds.
__device__ __forceinline__ uint32_t row_bcast(uint32_t v, int j) {
#define KVQ_RB(n) \
  case n: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x150 + n, 0xF, 0xF, false);
  switch (j) {
    KVQ_RB(0) KVQ_RB(1) KVQ_RB(2) KVQ_RB(3) KVQ_RB(4) KVQ_RB(5) KVQ_RB(6) KVQ_RB(7)
    KVQ_RB(8) KVQ_RB(9) KVQ_RB(10) KVQ_RB(11) KVQ_RB(12) KVQ_RB(13) KVQ_RB(14)
    default: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x150 + 15, 0xF, 0xF, false);
  }
#undef KVQ_RB
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_k32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_k16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a),
                                                   __builtin_bit_cast(bf16x4, b), c, 0, 0, 0);
}

struct MfParams {
  DecodeArgs a;
  int gt, n_hg;
  int tn;            // column tiles per unit (every wave computes each over its pages)
  ItemRule rule;     // work item size (see plan_items)
  int fused;         // merge split-K partials in the last workgroup (else a merge kernel)
  int whole;         // extend: items over whole sequences, streamed in sub-chunks
  float scale_log2;  // sm_scale * log2(e)
  int* prefix;       // [batch + 1]
  int* count;        // [batch * units] arrival counters, zero between calls
  float* part_ml;    // [items][tn * gt][2]
  float* part_acc;   // [items][tn * gt][D]
};

template <int QT, int D>
struct MfGeo {
  static constexpr int ESZ = (QT == QT_BF16) ? 2 : 1;
  static constexpr int NKS = D / 32;              // QK k-steps = scale blocks per row
  static constexpr int NT = D / 16;               // PV row tiles
  static constexpr int KDW = 2 * ESZ;             // dwords of a lane's 8 K elements
  // 8-bit codes: a lane loads 16 contiguous codes of its token per 64 elements
  // (one 16-byte load), and a cross-half lane swap hands every lane group
  // its 8 codes of each 32-element block; bf16: one 16-byte load per block
  static constexpr int KLD = (ESZ == 1) ? D / 64 : NKS;  // K loads per lane per page
  static constexpr int VDW = (D / 16) * ESZ / 4;  // dwords of a lane's V slice per token
  static constexpr int CODE = kPageSize * D * ESZ;
  static constexpr int SCL = qt_scaled(QT) ? kPageSize * NKS * 2 : 4;
};

template <int QT, int D>
struct PageRaw {
  using G = MfGeo<QT, D>;
  uint32_t k[G::KLD][4];
  uint32_t v[4][G::VDW];
  // K scales of tokens 4g .. 4g+3 (8 NKS bytes): dword j of them in lane
  // (j, g), fetched by the lanes of the row with a DPP row broadcast
  uint32_t ks;
  uint32_t vs[4];
};

template <int N, int AUX>
__device__ __forceinline__ void bload(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* o) {
  if constexpr (N == 4) {
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  } else if constexpr (N == 2) {
    const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX));
    o[0] = v.x; o[1] = v.y;
  } else if constexpr (N == 1) {
    o[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX);
  } else {
    static_assert(N == 8, "load width");
    bload<4, AUX>(r, off, o);
    bload<4, AUX>(r, off + 16, o + 4);
  }
}

// 4x4 byte transpose: out[c] byte r = in[r] byte c.
__device__ __forceinline__ void transpose4x4(const uint32_t* in, uint32_t* out) {
  const uint32_t t0 = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);
  const uint32_t t1 = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);
  const uint32_t t2 = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);
  const uint32_t t3 = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);
  out[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// EXT: extend attention (query rows are new tokens x heads, each with its own
// causal end); false: the decode, whose item end is uniform over the wave.
// TN: 16-column tiles per unit.  With TN = 2 every wave computes both tiles
// over its pages, so a page's loads and V dequantization serve 32 query rows
// (used with full tiles only: gt = 16, so a unit's column h is LDS column h).
// POL: the cache policy of the K/V loads -- non-temporal where each page is
// read by one work item (the decode; extend with few tile groups per kv
// head), the default where several items read it and can meet it in the L2.
// Two consecutive floats with one agent-scope 8-byte load (the split-K
// partials written by other workgroups).
__device__ __forceinline__ float2 load_agent2(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}

template <int QT, int D, bool EXT, int TN, bool SUB, int POL>
__global__ __launch_bounds__(kT) void gqa_mfma_kernel(MfParams p) {
  using Gm = MfGeo<QT, D>;
  constexpr int ESZ = Gm::ESZ, NKS = Gm::NKS, NT = Gm::NT, VDW = Gm::VDW, KLD = Gm::KLD;
  constexpr int CODE = Gm::CODE, SCL = Gm::SCL;
  using Raw = PageRaw<QT, D>;
  // page buffers per wave: NBUF pages' loads in flight while one is computed.
  // The decode runs one work item per compute unit, so one wave per SIMD:
  // three buffers (up to 256 VGPRs) keep more bytes in flight (57.0 against
  // 58.7 us per call for 262144 tokens at head_dim 256, 37.9 against 41.8
  // for 8 ragged contexts; four were slower than two).  Extend attention
  // keeps two, so that two waves of its two-tile items fit each SIMD.
  constexpr int NBUF = EXT ? 2 : 3;
  extern __shared__ int s_prefix[];  // [batch + 1]
  // per-wave (m, l) and O^T accumulators at the end of an item, or the merge's
  // chunk weights
  constexpr int kC = kN * TN;  // columns of a unit
  // (rows of the combine are D + 1 floats apart: the 16 lanes of a column
  // group write one element of 16 different rows, on 16 different banks)
  constexpr int kRow = D + 1;
  constexpr int kRed = (kW * kC * kRow > kMergeMaxWeights) ? kW * kC * kRow : kMergeMaxWeights;
  __shared__ float s_red[kRed];
  __shared__ float s_ml[kW][kC][2];
  __shared__ float s_hm[kC][2];
  __shared__ float s_wt[kW][kC];  // each wave's weight per column in the cross-wave merge
  __shared__ int s_wave[kW];
  __shared__ int s_last;

  const DecodeArgs& a = p.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g = lane >> 4;
  const int GT = p.gt;
  const int GTU = GT * TN;  // columns of a unit
  const int units = a.n_kv_heads * p.n_hg;
  const int G = a.n_q_heads / a.n_kv_heads;

  const int item_tokens = plan_items<kT>(a, p.rule, units, s_prefix, s_wave);
  const int total = s_prefix[a.batch];
  if (blockIdx.x == 0)
    for (int b = tid; b <= a.batch; b += kT) p.prefix[b] = s_prefix[b];
  for (int b = blockIdx.x; b < a.batch; b += gridDim.x) {
    if (s_prefix[b] != s_prefix[b + 1]) continue;
    // a sequence without work items (no valid length): its query rows, one
    // per head (decode) or per head of each new token (extend), are 0 / -inf
    int64_t r0 = (int64_t)b * a.n_q_heads, nr = a.n_q_heads;
    if (a.q_start) {
      r0 = (int64_t)a.q_start[b] * a.n_q_heads;
      nr = (int64_t)max(min(a.q_start[b + 1] - a.q_start[b], a.max_new), 0) * a.n_q_heads;
    }
    for (int64_t i = tid; i < nr * D; i += kT) a.out[r0 * D + i] = 0;
    if (a.lse)
      for (int64_t h = tid; h < nr; h += kT) a.lse[r0 + h] = -INFINITY;
  }

  // per-lane offsets inside a (page, kv head) chunk
  // K: token n16, elements 64 m + 16 g .. +15 (8-bit, + 64 m) or 32 ks + 8 g
  // .. +7 (bf16, + 64 ks bytes)
  const uint32_t koff = (uint32_t)(ESZ == 1 ? n16 * D + 16 * g : (n16 * D + 8 * g) * 2);
  const uint32_t voff = (uint32_t)((4 * g * D + (D / 16) * n16) * ESZ);       // + r D ESZ
  const uint32_t ksoff = (uint32_t)(8 * NKS * g + 4 * min(n16, 2 * NKS - 1));
  const int vblk = n16 * D / 512;                                             // V scale block
  const uint32_t vsoff = (uint32_t)(4 * g * NKS * 2 + (vblk * 2 & ~3));       // + r NKS 2
  const int vshift = (vblk & 1) * 16;
  const int64_t page_rows = (int64_t)a.n_kv_heads * kPageSize;

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    // ---- describe the item -------------------------------------------------------
    int lo = 0, hi = a.batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_prefix[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int rem = item - s_prefix[b];
    const int chunk = rem / units, u = rem - chunk * units;
    // Units are (kv head, tile of query rows).  Extend attention numbers them
    // tile-major, so the tiles of one kv head sit n_kv_heads items apart: with
    // 8 kv heads on the same XCD (blockIdx % 8), where they read the same
    // pages at about the same time through one L2.
    const int kvh = EXT ? u % a.n_kv_heads : u / p.n_hg;
    const int hg = EXT ? u / a.n_kv_heads : u - kvh * p.n_hg;
    const int L = clamped_len(a, b);
    const int nc = (L + item_tokens - 1) / item_tokens;
    const int t_item = chunk * item_tokens;
    int nt_item = min(item_tokens, L - t_item);
    // SUB: an extend item may span more pages than a wave's page-id list
    // holds (a whole sequence per item, see plan_decode); it is streamed in
    // sub-chunks of at most kMaxItemPages pages, carrying the softmax state
    // across them.  Otherwise an item is one sub-chunk.
    constexpr int kSubTokens = kMaxItemPages * kPageSize;
    // extend attention: a tile of query rows past the sequence's new tokens
    // has nothing to compute or write (uniform over the block; every chunk
    // of the tile skips, so its split-K counter stays untouched)
    const int col0 = hg * GTU;  // the unit's first column of the kv head's query rows
    if (EXT && col0 / G >= min(a.q_start[b + 1] - a.q_start[b], a.max_new)) continue;
    // this lane's query rows (one per tile) and the item tokens each may attend
    // to (the decode's: the item's own tokens, a wave-uniform bound)
    int64_t qrow_lane[TN];
    int col_end[TN];  // the item's tokens each column may attend to, from t_item
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int col = col0 + t * GT + n16;
      qrow_lane[t] = (n16 < GT) ? (EXT ? query_row(a, b, kvh, col, G)
                                       : (int64_t)b * a.n_q_heads + kvh * G + col)
                                : -1;
      col_end[t] = nt_item;
      if constexpr (EXT)
        col_end[t] = (n16 < GT) ? max(min(nt_item, query_end(a, b, L, col, G) - t_item), 0) : 0;
    }
    if constexpr (EXT) {
      // the item's tokens past every column's causal end are not streamed
      // (in a prefill, a tile near the start attends to a few pages only); an
      // item left with none still takes part in its unit's merge
      int e = col_end[0];
#pragma unroll
      for (int t = 1; t < TN; ++t) e = max(e, col_end[t]);
      // (token counts are exact in fp32)
      const float ef = stride_max<1>((float)e);
      nt_item = min(nt_item, (int)__int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(ef))));
    }
    const int nsub = SUB ? max((nt_item + kSubTokens - 1) / kSubTokens, 1) : 1;

    // The current sub-chunk: its first token t0, its tokens nt, each
    // column's limit within it, this wave's steps, and their page ids (lane
    // k holds the id of step k: page wave + 4k of the sub-chunk, at most 64
    // steps; -1 when masked or absent).  The stream runs a whole number of
    // NBUF-step rounds (at least one), so every path through it issues the
    // same loads.
    int t0, nt, nsteps, nst, pids;
    int col_lim[TN];
    auto set_sub = [&](int sub) {
      t0 = t_item + sub * kSubTokens;
      nt = min(kSubTokens, nt_item - sub * kSubTokens);
      const int np = (nt + kPageSize - 1) / kPageSize;
#pragma unroll
      for (int t = 0; t < TN; ++t) col_lim[t] = min(max(col_end[t] - sub * kSubTokens, 0), nt);
      nsteps = (np > wave) ? (np - wave + kW - 1) / kW : 0;  // pages of this wave
      nst = max((nsteps + NBUF - 1) / NBUF * NBUF, NBUF);
      pids = -1;
      if (lane < nsteps) {
        const int pi = wave + lane * kW;
        const int v = a.page_table[(int64_t)b * a.pt_stride + t0 / kPageSize + pi];
        pids = (v >= 0 && (int64_t)v < a.num_pages) ? v : -1;
      }
    };
    set_sub(0);
    // padded steps past the wave's pages are masked (id -1)
    auto pid_of = [&](int st) {
      const int v = __builtin_amdgcn_readlane(pids, min(st, 63));
      return st < nsteps ? v : -1;
    };

    // Q^T operands: qb[t][ks] = the query row of column n16 of tile t,
    // elements 32ks + 8g .. +7 (0 for padding columns)
    u32x4 qb[TN][NKS];
    {
      // the elements of block ks that lane group g holds in the K operand:
      // 32 ks + 8 g (bf16), or after the 8-bit lane swap 32 ks + (0, 16, 8, 24)[g]
      const int goff = (ESZ == 1) ? 16 * (g & 1) + 8 * (g >> 1) : 8 * g;
      // a padding column reads the unit's first row (it exists: units with no
      // row are skipped above) and zeroes it
      const int64_t row0 = EXT ? query_row(a, b, kvh, col0, G)
                               : (int64_t)b * a.n_q_heads + kvh * G + col0;
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const bool real = qrow_lane[t] >= 0;
        const uint16_t* qrow = a.q + (real ? qrow_lane[t] : row0) * D + goff;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 32 * ks);
          if (!real) v = u32x4{0, 0, 0, 0};
          qb[t][ks] = v;
        }
      }
    }

    // The loads of a page are issued on every path, never under a branch:
    // the hardware counts outstanding loads in issue order, and a load
    // skipped on one path would make the compiler wait for every load in
    // flight (the prefetch included) before the next compute.  A masked or
    // absent page (id -1) gets zero-length descriptors, whose loads return 0
    // without touching memory; its rows are never used.
    auto load_page = [&](int pid, Raw& R) {
      const int P = max(pid, 0);
      const int64_t row0 = (int64_t)P * page_rows + (int64_t)kvh * kPageSize;
      const int code_bytes = pid >= 0 ? CODE : 0;
      const auto rk = page_rsrc(a.k_pool + row0 * D * ESZ, code_bytes);
      const auto rv = page_rsrc(a.v_pool + row0 * D * ESZ, code_bytes);
#pragma unroll
      for (int m = 0; m < KLD; ++m) bload<4, POL>(rk, koff + 64 * m, R.k[m]);
#pragma unroll
      for (int r = 0; r < 4; ++r) bload<VDW, POL>(rv, voff + r * D * ESZ, R.v[r]);
      if constexpr (qt_scaled(QT)) {
        const auto rks = page_rsrc(a.k_scales + row0 * NKS, pid >= 0 ? SCL : 0);
        const auto rvs = page_rsrc(a.v_scales + row0 * NKS, pid >= 0 ? SCL : 0);
        R.ks = __builtin_amdgcn_raw_buffer_load_b32(rks, ksoff, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          R.vs[r] = __builtin_amdgcn_raw_buffer_load_b32(rvs, vsoff + r * NKS * 2, 0, 0);
      }
    };

    // ---- S^T = K Q^T of one page: log2-domain scores of tokens 4g .. 4g+3 of
    // the page for column n16 of each tile, -inf past the column's end or on
    // a masked page; ok: the token exists ---------------------------------------
    auto scores = [&](int st, int pid, const Raw& R, float (*s)[4], bool* ok) {
      if constexpr (QT == QT_BF16) {
        f32x4 S[TN];
#pragma unroll
        for (int t = 0; t < TN; ++t) S[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int t = 0; t < TN; ++t)
            S[t] = mfma_k32(u32x4{R.k[ks][0], R.k[ks][1], R.k[ks][2], R.k[ks][3]}, qb[t][ks], S[t]);
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[t][r] = S[t][r];
      } else if constexpr (!qt_scaled(QT)) {
        // cast codes (no scales): one product chain over the k-steps, the
        // codes handed to the lane groups as below
        f32x4 S[TN];
#pragma unroll
        for (int t = 0; t < TN; ++t) S[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const int m = ks >> 1;
          const auto x0 = __builtin_amdgcn_permlane32_swap(R.k[m][0], R.k[m][2], false, false);
          const auto x1 = __builtin_amdgcn_permlane32_swap(R.k[m][1], R.k[m][3], false, false);
          const uint32_t c0 = (ks & 1) ? x0[1] : x0[0], c1 = (ks & 1) ? x1[1] : x1[0];
          uint32_t kb[4];
          decode_dword_bf16x2<QT>(c0, kb);
          decode_dword_bf16x2<QT>(c1, kb + 2);
#pragma unroll
          for (int t = 0; t < TN; ++t)
            S[t] = mfma_k32(u32x4{kb[0], kb[1], kb[2], kb[3]}, qb[t][ks], S[t]);
        }
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[t][r] = S[t][r];
      } else {
        // one product tile per scale block, in groups of four live tiles
        constexpr int GS = NKS < 4 ? NKS : 4;
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[t][r] = 0.0f;
#pragma unroll
        for (int k0 = 0; k0 < NKS; k0 += GS) {
          f32x4 Sk[TN][GS];
#pragma unroll
          for (int k = 0; k < GS; ++k) {
            // block ks = 2m + j: lanes 0-31 hold 16 codes of block 2m, lanes
            // 32-63 of block 2m + 1; a swap of the upper half of one dword
            // pair with the lower half of the other gives every lane group 8
            // codes of each block (elements 32 ks + (0, 16, 8, 24)[g] ..)
            const int ks = k0 + k, m = ks >> 1;
            const auto x0 = __builtin_amdgcn_permlane32_swap(R.k[m][0], R.k[m][2], false, false);
            const auto x1 = __builtin_amdgcn_permlane32_swap(R.k[m][1], R.k[m][3], false, false);
            const uint32_t c0 = (ks & 1) ? x0[1] : x0[0], c1 = (ks & 1) ? x1[1] : x1[0];
            uint32_t kb[4];
            decode_dword_bf16x2<QT>(c0, kb);
            decode_dword_bf16x2<QT>(c1, kb + 2);
#pragma unroll
            for (int t = 0; t < TN; ++t)
              Sk[t][k] = mfma_k32(u32x4{kb[0], kb[1], kb[2], kb[3]}, qb[t][k0 + k],
                                  f32x4{0.f, 0.f, 0.f, 0.f});
          }
#pragma unroll
          for (int k = 0; k < GS; ++k) {
            const int ks = k0 + k;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              // scale (r, ks) is fp16 number r NKS + ks of the row's run
              const int idx = r * NKS + ks;
              const uint32_t w = row_bcast(R.ks, idx >> 1);
              const float sc = f16_bits_to_f32((uint16_t)(w >> ((idx & 1) * 16)));
#pragma unroll
              for (int t = 0; t < TN; ++t) s[t][r] = fmaf(sc, Sk[t][k][r], s[t][r]);
            }
          }
        }
      }
      const int tok0 = (wave + st * kW) * kPageSize + 4 * g;  // token of r = 0 in the item
      // ok: the token exists (its V rows are used, masked to zero otherwise);
      // a score is kept only below its column's end as well.  A lane's V
      // registers hold rows of other columns' products, so the V mask must
      // not depend on the column.  (Selects, not branches around the page's
      // work.)
      const int lim = pid >= 0 ? nt : 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) ok[r] = tok0 + r < lim;
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int slim = pid >= 0 ? col_lim[t] : 0;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s[t][r] = (tok0 + r < slim) ? s[t][r] * p.scale_log2 : -INFINITY;
      }
    };

    // ---- weights against the fixed reference, O^T += V^T P^T -------------------
    float mref[TN], lsum[TN], smax[TN];  // for column n16 of each tile (the same in every lane group)
    f32x4 acc[TN][NT];
    auto accumulate = [&](const Raw& R, const float (*s)[4], const bool* ok) {
      u32x2 pt[TN];
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          smax[t] = fmaxf(smax[t], s[t][r]);
          pr[r] = __builtin_amdgcn_exp2f(s[t][r] - mref[t]);  // 0 for a -inf score
          lsum[t] += pr[r];
        }
        pt[t] = u32x2{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])};
      }
      // tokens past the item end or on a masked page: codes and scale zeroed
      // (their probability is 0, but the slot may hold NaN codes)
      // (masks, not branches, so the page's work stays one scheduling region)
      uint32_t keep[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) keep[r] = ok[r] ? 0xffffffffu : 0u;
      if constexpr (QT == QT_BF16) {
        uint32_t w[4][VDW];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int k = 0; k < VDW; ++k) w[r][k] = R.v[r][k] & keep[r];
#pragma unroll
        for (int k = 0; k < VDW; ++k) {  // dword k holds dv 2k, 2k+1
          const u32x2 e0 = u32x2{__builtin_amdgcn_perm(w[1][k], w[0][k], 0x05040100u),
                                 __builtin_amdgcn_perm(w[3][k], w[2][k], 0x05040100u)};
          const u32x2 e1 = u32x2{__builtin_amdgcn_perm(w[1][k], w[0][k], 0x07060302u),
                                 __builtin_amdgcn_perm(w[3][k], w[2][k], 0x07060302u)};
#pragma unroll
          for (int t = 0; t < TN; ++t) {
            acc[t][2 * k] = mfma_k16(e0, pt[t], acc[t][2 * k]);
            acc[t][2 * k + 1] = mfma_k16(e1, pt[t], acc[t][2 * k + 1]);
          }
        }
      } else {
        float sv[4];
        uint32_t w[4][VDW];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sv[r] = qt_scaled(QT) ? f16_bits_to_f32((uint16_t)((R.vs[r] >> vshift) & keep[r])) : 1.0f;
#pragma unroll
          for (int k = 0; k < VDW; ++k) w[r][k] = R.v[r][k] & keep[r];
        }
#pragma unroll
        for (int k = 0; k < VDW; ++k) {  // dword k holds dv 4k .. 4k+3 of each token
          uint32_t col[4];
          const uint32_t in[4] = {w[0][k], w[1][k], w[2][k], w[3][k]};
          transpose4x4(in, col);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            u32x2 e;
            if constexpr (qt_scaled(QT)) {
              float f[4];
              decode_dword<QT>(col[c], f);
              e = u32x2{pack_bf16x2(f[0] * sv[0], f[1] * sv[1]),
                        pack_bf16x2(f[2] * sv[2], f[3] * sv[3])};
            } else {  // cast codes: exact bf16 pairs of tokens (0, 1) and (2, 3)
              uint32_t pr2[2];
              decode_dword_bf16x2<QT>(col[c], pr2);
              e = u32x2{pr2[0], pr2[1]};
            }
#pragma unroll
            for (int t = 0; t < TN; ++t) acc[t][4 * k + c] = mfma_k16(e, pt[t], acc[t][4 * k + c]);
          }
        }
      }
    };

    // ---- stream this wave's pages, NBUF pages' loads in flight ---------------------
    // The softmax reference of a column stays fixed over the pass: the largest
    // score of the wave's first page (0 when it has none).  Weights 2^(s -
    // mref) then need no running-max update, no cross-lane reduction and no
    // rescaling of the accumulators.  A pass whose largest score ends up more
    // than 2^64 away from the reference (the weights could overflow, or every
    // weight underflow) is streamed again with that score as the reference.
    Raw R[NBUF];
    float M[TN];  // largest score of column n16 of each tile over the wave's pages
    for (int pass = 0;; ++pass) {
      for (int sub = 0; sub < nsub; ++sub) {
        if (sub > 0 || (pass > 0 && nsub > 1)) set_sub(sub);
#pragma unroll
        for (int k = 0; k < NBUF; ++k) load_page(pid_of(k), R[k]);
        if (pass == 0 && sub == 0) {
          float s0[TN][4];
          bool ok0[4];
          scores(0, pid_of(0), R[0], s0, ok0);
#pragma unroll
          for (int t = 0; t < TN; ++t) {
            float x = fmaxf(fmaxf(s0[t][0], s0[t][1]), fmaxf(s0[t][2], s0[t][3]));
            x = max_xor32(max_xor16(x));
            mref[t] = (x == -INFINITY) ? 0.0f : x;
          }
        }
        if (sub == 0) {
#pragma unroll
          for (int t = 0; t < TN; ++t) {
            lsum[t] = 0.0f;
            smax[t] = -INFINITY;
#pragma unroll
            for (int i = 0; i < NT; ++i) acc[t][i] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
        for (int st = 0; st < nst; st += NBUF) {
#pragma unroll
          for (int k = 0; k < NBUF; ++k) {
            float s[TN][4];
            bool ok[4];
            scores(st + k, pid_of(st + k), R[k], s, ok);
            accumulate(R[k], s, ok);
            load_page(pid_of(st + k + NBUF), R[k]);
          }
        }
      }
      bool redo = false;
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        M[t] = max_xor32(max_xor16(smax[t]));
        redo |= M[t] != -INFINITY && (M[t] > mref[t] + 64.0f || M[t] < mref[t] - 64.0f);
      }
      if (!__builtin_amdgcn_ballot_w64(redo)) break;
#pragma unroll
      for (int t = 0; t < TN; ++t) mref[t] = (M[t] == -INFINITY) ? 0.0f : M[t];
    }
    // a column with no valid token here contributes nothing to the merges
    float m[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) m[t] = (M[t] == -INFINITY) ? -INFINITY : mref[t];

    // ---- merge the four waves ---------------------------------------------------------
#pragma unroll
    for (int t = 0; t < TN; ++t) lsum[t] = sum_xor32(sum_xor16(lsum[t]));
    __syncthreads();  // s_red / s_ml of the previous item are free
    // O^T tile i, lane (column n16, group g), row 4g + r is dv (D/16)(4g + r) + i;
    // LDS column t kN + n16 (= the unit's column: gt = 16 whenever TN > 1)
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      float* dst = s_red + (wave * kC + t * kN + n16) * kRow;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < NT; ++i) dst[(D / 16) * (4 * g + r) + i] = acc[t][i][r];
      if (g == 0) {
        s_ml[wave][t * kN + n16][0] = m[t];
        s_ml[wave][t * kN + n16][1] = lsum[t];
      }
    }
    __syncthreads();
    if (tid < kC) {
      float M = s_ml[0][tid][0];
#pragma unroll
      for (int w = 1; w < kW; ++w) M = fmaxf(M, s_ml[w][tid][0]);
      float Ls = 0.0f;
#pragma unroll
      for (int w = 0; w < kW; ++w) {
        const float wt = exp2_rel(s_ml[w][tid][0], M);
        s_wt[w][tid] = wt;
        Ls += wt * s_ml[w][tid][1];
      }
      s_hm[tid][0] = M;
      s_hm[tid][1] = Ls;
    }
    __syncthreads();
    // kR output elements per thread per round: every LDS read of a round is
    // issued before the first is used (one at a time, each exp and read
    // waited on the one before: about 2.8 us per item at head_dim 256)
    constexpr int kR = 4;
    for (int idx0 = tid; idx0 < GTU * D; idx0 += kR * kT) {
      float x[kR][kW], wt[kR][kW], Mr[kR], Lr[kR];
      int hr[kR], dr[kR];
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int idx = min(idx0 + r * kT, GTU * D - 1);
        hr[r] = idx / D;
        dr[r] = idx - hr[r] * D;
        Mr[r] = s_hm[hr[r]][0];
        Lr[r] = s_hm[hr[r]][1];
#pragma unroll
        for (int w = 0; w < kW; ++w) {
          x[r][w] = s_red[(w * kC + hr[r]) * kRow + dr[r]];
          wt[r][w] = s_wt[w][hr[r]];
        }
      }
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        if (idx0 + r * kT >= GTU * D) continue;
        const int h = hr[r], d = dr[r];
        const float M = Mr[r];
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < kW; ++w) v += wt[r][w] * x[r][w];
        if (nc == 1) {
          const float Ls = Lr[r];
          const int64_t orow = EXT ? query_row(a, b, kvh, col0 + h, G)
                                   : (int64_t)b * a.n_q_heads + kvh * G + col0 + h;
          if (orow >= 0) {
            a.out[orow * D + d] = (uint16_t)bf16_rne(Ls > 0.0f ? v / Ls : 0.0f);
            if (d == 0 && a.lse) a.lse[orow] = (M == -INFINITY) ? -INFINITY : (M + log2f(Ls)) * kLn2;
          }
        } else {
          store_agent(&p.part_acc[((int64_t)item * GTU + h) * D + d], v);
          if (d == 0) {
            store_agent(&p.part_ml[((int64_t)item * GTU + h) * 2 + 0], M);
            store_agent(&p.part_ml[((int64_t)item * GTU + h) * 2 + 1], Lr[r]);
          }
        }
      }
    }

    if (nc > 1 && p.fused) {
      // ---- the last item of this (sequence, kv head, head group) merges ---------
      // Ordering (gfx950): the partials went out as agent-scope stores,
      // which write through the L2 to the cross-XCD coherence point; the
      // vmcnt(0) wait returns once each is acknowledged there, before the
      // barrier and thread 0's agent-scope increment.  The workgroup that
      // reads the final count issues its agent-scope loads (which bypass the
      // non-coherent caches) only after the increment has returned, so they
      // see every chunk's partials.  An acquire-release increment gives the
      // same order through an L2 write-back and invalidate and cost about
      // 1 us per call.
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) {
        const int old = __hip_atomic_fetch_add(&p.count[(int64_t)b * units + u], 1,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (old == nc - 1);
      }
      __syncthreads();
      if (s_last) {
        // Each thread merges kE consecutive elements of one column straight
        // from global memory (agent-scope loads, as the partials were
        // stored): every chunk's m for the maximum and the first kG chunks'
        // (m, l) and rows are requested together, later chunks kG at a time.
        // No LDS, no barrier.
        const int first = s_prefix[b] + u;  // item of chunk c: first + c * units
        const int64_t cstride = (int64_t)units * GTU * D;  // floats between chunks' rows
        const int64_t mstride = (int64_t)units * GTU * 2;  // ... and (m, l) pairs
        constexpr int kE = 16, kG = 4;
        for (int w0 = tid; w0 < GTU * (D / kE); w0 += kT) {
          const int h = w0 / (D / kE), d0 = (w0 - h * (D / kE)) * kE;
          const float* ml = p.part_ml + ((int64_t)first * GTU + h) * 2;
          const float* src = p.part_acc + ((int64_t)first * GTU + h) * D + d0;
          float2 mlc[kG], x[kG][kE / 2];
          auto load_group = [&](int c0) {
#pragma unroll
            for (int j = 0; j < kG; ++j) {
              const bool in = c0 + j < nc;
              mlc[j] = in ? load_agent2(ml + (c0 + j) * mstride) : make_float2(-INFINITY, 0.0f);
#pragma unroll
              for (int q = 0; q < kE / 2; ++q)
                x[j][q] = in ? load_agent2(src + (c0 + j) * cstride + 2 * q) : make_float2(0.0f, 0.0f);
            }
          };
          load_group(0);
          float M = -INFINITY;
          for (int c0 = 0; c0 < nc; c0 += 16) {
            float mc[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) mc[j] = (c0 + j < nc) ? load_agent(ml + (c0 + j) * mstride) : -INFINITY;
#pragma unroll
            for (int j = 0; j < 16; ++j) M = fmaxf(M, mc[j]);
          }
          float v[kE], Ls = 0.0f;
#pragma unroll
          for (int e = 0; e < kE; ++e) v[e] = 0.0f;
          for (int c0 = 0; c0 < nc; c0 += kG) {
            if (c0 > 0) load_group(c0);
#pragma unroll
            for (int j = 0; j < kG; ++j) {
              const float w = exp2_rel(mlc[j].x, M);  // 0 past the last chunk (m = -inf)
              Ls += w * mlc[j].y;
#pragma unroll
              for (int q = 0; q < kE / 2; ++q) {
                v[2 * q] += w * x[j][q].x;
                v[2 * q + 1] += w * x[j][q].y;
              }
            }
          }
          const int64_t orow = EXT ? query_row(a, b, kvh, col0 + h, G)
                                   : (int64_t)b * a.n_q_heads + kvh * G + col0 + h;
          if (orow >= 0) {
            uint32_t* o = reinterpret_cast<uint32_t*>(a.out + orow * D + d0);
#pragma unroll
            for (int q = 0; q < kE / 2; ++q)
              o[q] = pack_bf16x2(Ls > 0.0f ? v[2 * q] / Ls : 0.0f, Ls > 0.0f ? v[2 * q + 1] / Ls : 0.0f);
            if (d0 == 0 && a.lse)
              a.lse[orow] = (M == -INFINITY) ? -INFINITY : (M + log2f(Ls)) * kLn2;
          }
        }
        if (tid == 0)
          __hip_atomic_store(&p.count[(int64_t)b * units + u], 0, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

template <int QT, int D>
hipError_t launch_d(const MfParams& mp, int grid, hipStream_t s) {
  const size_t dyn = (size_t)(mp.a.batch + 1) * sizeof(int);
  // Extend: with at least kSharedTileGroups tile groups per kv head, every
  // page is read by that many work items on one XCD, and loads with the
  // default policy let them meet it in the L2 (64 new tokens, 4 groups:
  // 207 against 225 us, HBM traffic 1.44x instead of 2.08x); with fewer the
  // non-temporal loads are faster (8 new tokens: 69 against 75 us).  Whole-
  // sequence items come from long prefills, with many groups.
  constexpr int NT = kNonTemporal;
  const bool shared = mp.n_hg >= kSharedTileGroups;
  if (mp.a.q_start && mp.tn == 2) {
    if constexpr (D <= 128) {
      if (mp.whole) gqa_mfma_kernel<QT, D, true, 2, true, 0><<<grid, kT, dyn, s>>>(mp);
      else if (shared) gqa_mfma_kernel<QT, D, true, 2, false, 0><<<grid, kT, dyn, s>>>(mp);
      else gqa_mfma_kernel<QT, D, true, 2, false, NT><<<grid, kT, dyn, s>>>(mp);
    } else {
      return hipErrorInvalidValue;  // the planner uses two tiles only up to head_dim 128
    }
  } else if (mp.a.q_start) {
    if (mp.whole) gqa_mfma_kernel<QT, D, true, 1, true, 0><<<grid, kT, dyn, s>>>(mp);
    else if (shared) gqa_mfma_kernel<QT, D, true, 1, false, 0><<<grid, kT, dyn, s>>>(mp);
    else gqa_mfma_kernel<QT, D, true, 1, false, NT><<<grid, kT, dyn, s>>>(mp);
  } else {
    gqa_mfma_kernel<QT, D, false, 1, false, NT><<<grid, kT, dyn, s>>>(mp);
  }
  return hipGetLastError();
}

template <int QT>
hipError_t launch_q(const MfParams& mp, int grid, hipStream_t s) {
  switch (mp.a.head_dim_qk) {
    case 64: return launch_d<QT, 64>(mp, grid, s);
    case 128: return launch_d<QT, 128>(mp, grid, s);
    default: return launch_d<QT, 256>(mp, grid, s);
  }
}

}  // namespace

hipError_t launch_gqa_mfma_decode(const DecodeArgs& a, const DecodePlan& plan, int num_cus,
                                  hipStream_t s) {
  char* ws = static_cast<char*>(a.workspace);
  MfParams mp;
  mp.a = a;
  mp.gt = plan.gt;
  mp.n_hg = plan.n_hg;
  mp.tn = plan.tn;
  mp.rule = ItemRule{plan.step, plan.min_pages, plan.cap_pages, plan.target};
  mp.fused = plan.fused_merge ? 1 : 0;
  mp.whole = plan.whole ? 1 : 0;
  mp.scale_log2 = a.sm_scale * kLog2e;
  mp.prefix = reinterpret_cast<int*>(ws + plan.off_prefix);
  mp.count = reinterpret_cast<int*>(ws + plan.off_count);
  mp.part_ml = reinterpret_cast<float*>(ws + plan.off_ml);
  mp.part_acc = reinterpret_cast<float*>(ws + plan.off_acc);
  int64_t grid = plan.target;
  if (grid > plan.max_items) grid = plan.max_items;
  if (a.items_hint > 0 && grid > a.items_hint) grid = a.items_hint;  // exact from host lengths
  if (grid < 1) grid = 1;
  hipError_t e;
  switch (a.qtype) {
    case QT_BF16: e = launch_q<QT_BF16>(mp, (int)grid, s); break;
    case QT_FP8: e = launch_q<QT_FP8>(mp, (int)grid, s); break;
    case QT_FP8C: e = launch_q<QT_FP8C>(mp, (int)grid, s); break;
    case QT_BF8C: e = launch_q<QT_BF8C>(mp, (int)grid, s); break;
    default: e = launch_q<QT_Q8>(mp, (int)grid, s); break;
  }
  if (e != hipSuccess || plan.fused_merge) return e;
  return launch_gqa_merge(a, plan, s);
}

}  // namespace kvq
