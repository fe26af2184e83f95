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
// stores (m, l, acc) for every head and mla_merge_kernel combines them.
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
constexpr int kSlack = 64;            // log2-domain headroom above the softmax reference

__device__ __forceinline__ int vt_index(int d, int pos) { return d * kVR + (d >> 4) * 8 + pos; }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// D = A B + C for a 16x32 A (lane l: row l%16, k = 8(l/16) .. +7), a 32x16 B
// (lane l: column l%16, the same k) and a 16x16 fp32 D (lane l: column l%16,
// rows 4(l/16) .. +3).
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

struct MlaParams {
  DecodeArgs a;
  int item_tokens;   // a multiple of kTile
  float scale_log2;  // sm_scale * log2(e)
  int* prefix;       // [batch + 1] items before each sequence (written by block 0)
  float* part_ml;    // [items][n_q_heads][2]  (log2-domain max, sum)
  float* part_acc;   // [items][n_q_heads][512]
};

template <int QT>
struct MlaGeo {
  static constexpr int ESZ = (QT == QT_BF16) ? 2 : 1;
  static constexpr int ROWB = kDqk * ESZ;           // code bytes per token row
  static constexpr int PAGEB = kPageSize * ROWB;    // code bytes per page
  static constexpr int SCLB = kPageSize * kNB * 2;  // scale bytes per page
  static constexpr int VW = 4 * ESZ;                // dwords of 16 V-part elements
  static constexpr int RW = 2 * ESZ;                // dwords of 8 rope elements
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
};

template <int N>
__device__ __forceinline__ void buf_load_dw(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t* o) {
  if constexpr (N == 8) {
    buf_load_dw<4>(rs, off, o);
    buf_load_dw<4>(rs, off + 16, o + 4);
  } else if constexpr (N == 4) {
    const u32x4 v = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kNonTemporal));
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  } else {
    static_assert(N == 2, "load width");
    const u32x2 v = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kNonTemporal));
    o[0] = v.x; o[1] = v.y;
  }
}

// Codes of one dword (four 8-bit codes, or two bf16) times the block scale,
// rounded once to bf16 pairs (the product is exact in fp32).
template <int QT>
__device__ __forceinline__ void dequant_dword(uint32_t w, float s, uint32_t* o) {
  if constexpr (QT == QT_BF16) {
    o[0] = w;
  } else {
    float f[4];
    decode_dword<QT>(w, f);
    o[0] = pack_bf16x2(f[0] * s, f[1] * s);
    o[1] = pack_bf16x2(f[2] * s, f[3] * s);
  }
}

__device__ __forceinline__ float scale_half(uint32_t w, int shift) {
  return f16_bits_to_f32((uint16_t)(w >> shift));
}

template <int QT>
__global__ __launch_bounds__(kT) void mla_decode_kernel(MlaParams p) {
  using Gm = MlaGeo<QT>;
  constexpr int ESZ = Gm::ESZ, ROWB = Gm::ROWB, PAGEB = Gm::PAGEB, SCLB = Gm::SCLB;
  constexpr int VW = Gm::VW, RW = Gm::RW;
  constexpr int EPD = (QT == QT_BF16) ? 1 : 2;  // bf16 pairs per code dword
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][kTile * kKS];
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[2][kVtElems];
  __shared__ int s_wave[kW];
  __shared__ int s_flag[3];  // per-tile restart votes, rotating
  extern __shared__ int s_prefix[];  // [batch + 1]

  const DecodeArgs& a = p.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g = lane >> 4;
  const int Hq = a.n_q_heads;

  build_prefix<kT>(a, p.item_tokens, 1, s_prefix, s_wave);
  const int total = s_prefix[a.batch];
  if (blockIdx.x == 0)
    for (int b = tid; b <= a.batch; b += kT) p.prefix[b] = s_prefix[b];
  // a sequence with no valid length has no items: its output is 0, lse -inf
  for (int b = blockIdx.x; b < a.batch; b += gridDim.x) {
    if (s_prefix[b] != s_prefix[b + 1]) continue;
    for (int i = tid; i < Hq * kDv; i += kT) a.out[(int64_t)b * Hq * kDv + i] = 0;
    if (a.lse)
      for (int h = tid; h < Hq; h += kT) a.lse[(int64_t)b * Hq + h] = -INFINITY;
  }

  // ---- loader geometry (fixed per thread) ---------------------------------------
  const int q4 = tid >> 5, u = tid & 31;  // V part: token quad, 16-element unit
  const int rt = tid >> 3, p8 = tid & 7;  // rope: token, 8-element unit
  const int wpage = wave >> 1;            // page of the tile this wave's loads touch
  uint32_t voff[4], soff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tip = (4 * q4 + i) & (kPageSize - 1);
    voff[i] = (uint32_t)(tip * ROWB + u * 16 * ESZ);
    soff[i] = (uint32_t)(tip * kNB * 2 + (u >> 2) * 4);
  }
  const uint32_t roff = (uint32_t)((rt & (kPageSize - 1)) * ROWB + (kDv + 8 * p8) * ESZ);
  const uint32_t rsoff = (uint32_t)((rt & (kPageSize - 1)) * kNB * 2 + (kDv / 32) * 2);
  const int vshift = ((u >> 1) & 1) * 16, rshift = (p8 >> 2) * 16;
  // position of the quad's first token in a V^T row: S^T hands lane group g
  // the tokens 4g..4g+3 of each 16-token half; they become k slots 8g..8g+7
  const int vpos = (q4 < 4) ? 8 * q4 : 8 * (q4 - 4) + 4;

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    // ---- describe the item (uniform over the block) ------------------------------
    int lo = 0, hi = a.batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_prefix[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int chunk = item - s_prefix[b];
    const int L = clamped_len(a, b);
    const int nc = (L + p.item_tokens - 1) / p.item_tokens;
    const int t0 = chunk * p.item_tokens;
    const int nt = min(p.item_tokens, L - t0);
    const int ntiles = (nt + kTile - 1) / kTile;
    const int npages = (nt + kPageSize - 1) / kPageSize;

    // page ids of the item: lane k holds page column t0/16 + k; masked -> -1
    int pid = -1;
    if (lane < npages) {
      const int v = a.page_table[(int64_t)b * a.pt_stride + t0 / kPageSize + lane];
      pid = (v >= 0 && (int64_t)v < a.num_pages) ? v : -1;
    }

    // this wave's 32 query heads as MFMA B operands: qr[ht][ks] holds, for
    // head 32w + 16ht + (l%16), elements 32ks + 8(l/16) .. +7
    u32x4 qr[2][kNB];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const int h = 32 * wave + 16 * ht + n16;
      const uint16_t* qrow = a.q + ((int64_t)b * Hq + (h < Hq ? h : 0)) * kDqk + 8 * g;
#pragma unroll
      for (int ks = 0; ks < kNB; ++ks) {
        u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 32 * ks);
        if (h >= Hq) v = u32x4{0, 0, 0, 0};
        qr[ht][ks] = v;
      }
    }

    auto load_tile = [&](int j, MlaRaw<QT>& R) {
      const int P = max(__builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(pid, 2 * j + wpage)), 0);
      const auto rc = page_rsrc(a.k_pool + (int64_t)P * PAGEB, PAGEB);
#pragma unroll
      for (int i = 0; i < 4; ++i) buf_load_dw<VW>(rc, voff[i], R.v[i]);
      buf_load_dw<RW>(rc, roff, R.r);
      if constexpr (QT != QT_BF16) {
        const auto rs = page_rsrc(a.k_scales + (int64_t)P * (SCLB / 2), SCLB);
#pragma unroll
        for (int i = 0; i < 4; ++i) R.vs[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, soff[i], 0, 0);
        R.rs = __builtin_amdgcn_raw_buffer_load_b32(rs, rsoff, 0, 0);
      }
    };

    // dequantize a loaded tile into LDS buffer `buf`, four elements at a
    // time for the thread's four tokens; rows of masked pages or past the
    // item end are written as zeros
    auto store_tile = [&](int j, const MlaRaw<QT>& R, int buf) {
      uint16_t* K = s_k[buf];
      uint16_t* Vt = s_vt[buf];
      const bool page_ok = __builtin_amdgcn_readlane(pid, 2 * j + wpage) >= 0;
      float sv[4];
      bool ok[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ok[i] = page_ok && (kTile * j + 4 * q4 + i < nt);
        sv[i] = (QT == QT_BF16) ? 1.0f : scale_half(R.vs[i], vshift);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {  // elements 16u + 4k .. +3
        uint32_t pr[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (QT == QT_BF16) {
            pr[i][0] = R.v[i][2 * k];
            pr[i][1] = R.v[i][2 * k + 1];
          } else {
            dequant_dword<QT>(R.v[i][k], sv[i], pr[i]);
          }
          pr[i][0] = ok[i] ? pr[i][0] : 0u;
          pr[i][1] = ok[i] ? pr[i][1] : 0u;
          *reinterpret_cast<u32x2*>(K + (4 * q4 + i) * kKS + 16 * u + 4 * k) = u32x2{pr[i][0], pr[i][1]};
        }
        // V^T: element d of the four tokens as two bf16 pairs
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          const uint32_t w01 = __builtin_amdgcn_perm(pr[1][e >> 1], pr[0][e >> 1], sel);
          const uint32_t w23 = __builtin_amdgcn_perm(pr[3][e >> 1], pr[2][e >> 1], sel);
          *reinterpret_cast<u32x2*>(Vt + vt_index(16 * u + 4 * k + e, vpos)) = u32x2{w01, w23};
        }
      }
      {
        const bool okr = page_ok && (kTile * j + rt < nt);
        const float s = (QT == QT_BF16) ? 1.0f : scale_half(R.rs, rshift);
        uint32_t rw[4];
#pragma unroll
        for (int k = 0; k < RW; ++k) dequant_dword<QT>(R.r[k], s, &rw[k * EPD]);
#pragma unroll
        for (int k = 0; k < 4; ++k) rw[k] = okr ? rw[k] : 0u;
        *reinterpret_cast<u32x4*>(K + rt * kKS + kDv + 8 * p8) = u32x4{rw[0], rw[1], rw[2], rw[3]};
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

    auto compute = [&](int j, int buf, int fslot) {
      const uint16_t* K = s_k[buf];
      const uint16_t* Vt = s_vt[buf];
      // S^T = K Q^T: lane l holds, for head 16ht + l%16, tokens 16tt + 4g .. +3
      f32x4 S[2][2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) S[tt][0] = S[tt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kNB; ++ks)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const u32x4 A = *reinterpret_cast<const u32x4*>(K + (16 * tt + n16) * kKS + 32 * ks + 8 * g);
          S[tt][0] = mfma16(A, qr[0][ks], S[tt][0]);
          S[tt][1] = mfma16(A, qr[1][ks], S[tt][1]);
        }
      const bool ok0 = __builtin_amdgcn_readlane(pid, 2 * j) >= 0;
      const bool ok1 = __builtin_amdgcn_readlane(pid, 2 * j + 1) >= 0;
      u32x4 pk[2];
      bool over = false;
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        float sc[8], t = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tok = kTile * j + 16 * tt + 4 * g + r;
            const bool ok = (tt ? ok1 : ok0) && tok < nt;
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
      // O^T += V^T P^T
#pragma unroll
      for (int dt = 0; dt < kDv / 16; ++dt) {
        const u32x4 A = *reinterpret_cast<const u32x4*>(Vt + vt_index(16 * dt + n16, 8 * g));
        acc[dt][0] = mfma16(A, pk[0], acc[dt][0]);
        acc[dt][1] = mfma16(A, pk[1], acc[dt][1]);
      }
    };

    MlaRaw<QT> R;
    while (true) {  // passes over the item (a second one only after a restart)
#pragma unroll
      for (int dt = 0; dt < kDv / 16; ++dt) {
        acc[dt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc[dt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      lsum[0] = lsum[1] = 0.0f;
      load_tile(0, R);
      __syncthreads();  // earlier reads of both buffers and of the votes are done
      if (tid < 3) s_flag[tid] = 0;
      store_tile(0, R, 0);
      if (ntiles > 1) load_tile(1, R);
      __syncthreads();
      // Tile j votes into slot j % 3 and is decided after its barrier.  The
      // slot of tile j+1 is cleared before that barrier: its last readers
      // (tile j-2's decision) are past barrier j-1, its writers after j.
      bool restart = false;
      for (int j = 0, slot = 0; j < ntiles; ++j) {
        const int next = (slot == 2) ? 0 : slot + 1;
        compute(j, j & 1, slot);
        if (j + 1 < ntiles) {
          store_tile(j + 1, R, (j + 1) & 1);
          if (j + 2 < ntiles) load_tile(j + 2, R);
        }
        if (tid == 0) s_flag[next] = 0;
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
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const float Ls = sum_xor32(sum_xor16(lsum[ht]));
      const int h = 32 * wave + 16 * ht + n16;
      if (h >= Hq) continue;
      if (nc == 1) {
        const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
        uint16_t* orow = a.out + ((int64_t)b * Hq + h) * kDv + 4 * g;
#pragma unroll
        for (int dt = 0; dt < kDv / 16; ++dt) {
          const f32x4 v = acc[dt][ht];
          *reinterpret_cast<u32x2*>(orow + 16 * dt) =
              u32x2{pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv)};
        }
        if (g == 0 && a.lse)
          a.lse[(int64_t)b * Hq + h] = (mref[ht] == -INFINITY) ? -INFINITY : (mref[ht] + log2f(Ls)) * kLn2;
      } else {
        float* prow = p.part_acc + ((int64_t)item * Hq + h) * kDv + 4 * g;
#pragma unroll
        for (int dt = 0; dt < kDv / 16; ++dt) *reinterpret_cast<f32x4*>(prow + 16 * dt) = acc[dt][ht];
        if (g == 0) {
          p.part_ml[((int64_t)item * Hq + h) * 2 + 0] = mref[ht];
          p.part_ml[((int64_t)item * Hq + h) * 2 + 1] = Ls;
        }
      }
    }
  }
}

// ---- split-K merge -------------------------------------------------------------------
// Block = (sequence b, head h, 32-column slice); 8 groups of 32 threads take
// every 8th chunk.  O = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c.
constexpr int kMergeCols = 32;
constexpr int kMergeGroups = 8;

__global__ __launch_bounds__(kMergeCols * kMergeGroups) void mla_merge_kernel(MlaParams p) {
  const DecodeArgs& a = p.a;
  const int Hq = a.n_q_heads;
  constexpr int kSlices = kDv / kMergeCols;
  const int slice = blockIdx.x % kSlices;
  const int bh = blockIdx.x / kSlices;
  const int h = bh % Hq, b = bh / Hq;
  const int first = p.prefix[b];
  const int nc = p.prefix[b + 1] - first;
  if (nc <= 1) return;  // written by the decode kernel itself
  __shared__ float s_w[kMlaMaxChunks];
  __shared__ float s_red[kMergeGroups][kMergeCols];
  __shared__ float s_ML[2];
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < 64) {
    float M = -INFINITY;
    for (int c = lane; c < nc; c += 64) M = fmaxf(M, p.part_ml[((int64_t)(first + c) * Hq + h) * 2]);
    M = stride_max<1>(M);
    float Ls = 0.0f;
    for (int c = lane; c < nc; c += 64) {
      const float* ml = p.part_ml + ((int64_t)(first + c) * Hq + h) * 2;
      const float w = exp2_rel(ml[0], M);
      s_w[c] = w;
      Ls += w * ml[1];
    }
    Ls = stride_sum<1>(Ls);
    if (lane == 0) {
      s_ML[0] = M;
      s_ML[1] = Ls;
    }
  }
  __syncthreads();
  const int grp = tid / kMergeCols, j = tid % kMergeCols;
  const int d = slice * kMergeCols + j;
  const float* src = p.part_acc + ((int64_t)first * Hq + h) * kDv + d;
  const int64_t cstride = (int64_t)Hq * kDv;
  float v = 0.0f;
  int c = grp;
  for (; c + 3 * kMergeGroups < nc; c += 4 * kMergeGroups) {
    const float x0 = src[(int64_t)c * cstride];
    const float x1 = src[(int64_t)(c + kMergeGroups) * cstride];
    const float x2 = src[(int64_t)(c + 2 * kMergeGroups) * cstride];
    const float x3 = src[(int64_t)(c + 3 * kMergeGroups) * cstride];
    v += s_w[c] * x0 + s_w[c + kMergeGroups] * x1 + s_w[c + 2 * kMergeGroups] * x2 +
         s_w[c + 3 * kMergeGroups] * x3;
  }
  for (; c < nc; c += kMergeGroups) v += s_w[c] * src[(int64_t)c * cstride];
  s_red[grp][j] = v;
  __syncthreads();
  if (tid < kMergeCols) {
    float t = 0.0f;
#pragma unroll
    for (int k = 0; k < kMergeGroups; ++k) t += s_red[k][tid];
    const float M = s_ML[0], Ls = s_ML[1];
    const int64_t orow = (int64_t)b * Hq + h;
    a.out[orow * kDv + d] = (uint16_t)bf16_rne(Ls > 0.0f ? t / Ls : 0.0f);
    if (d == 0 && a.lse) a.lse[orow] = (M == -INFINITY) ? -INFINITY : (M + log2f(Ls)) * kLn2;
  }
}

template <int QT>
hipError_t launch_q(const MlaParams& mp, int grid, int merge_grid, hipStream_t s) {
  const size_t dyn = (size_t)(mp.a.batch + 1) * sizeof(int);
  mla_decode_kernel<QT><<<grid, kT, dyn, s>>>(mp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || merge_grid == 0) return e;
  mla_merge_kernel<<<merge_grid, kMergeCols * kMergeGroups, 0, s>>>(mp);
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
  mp.part_acc = reinterpret_cast<float*>(ws + plan.off_acc);
  int64_t grid = num_cus;  // one workgroup per CU fits the tiles' LDS
  if (grid > plan.max_items) grid = plan.max_items;
  if (grid < 1) grid = 1;
  const int64_t max_chunks = (a.max_pages + plan.item_pages - 1) / plan.item_pages;
  const int merge_grid = (max_chunks > 1) ? a.batch * a.n_q_heads * (kDv / kMergeCols) : 0;
  switch (a.qtype) {
    case QT_BF16: return launch_q<QT_BF16>(mp, (int)grid, merge_grid, s);
    case QT_FP8: return launch_q<QT_FP8>(mp, (int)grid, merge_grid, s);
    default: return launch_q<QT_Q8>(mp, (int)grid, merge_grid, s);
  }
}

}  // namespace kvq
