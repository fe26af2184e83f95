// kvq_decode.hip -- paged decode attention over separate K/V pools (GQA):
// split-K over page chunks with an in-kernel log-sum-exp merge (gfx950, VALU).
//
// Sources: [PR103] "feat(kvcache): 8-bit KV cache (q8_0 / fp8_e4m3) behind
// --kv-cache-dtype" §What (dequant inside the attention kernels behind a QUANT
// switch; the scale varies along head_dim, the reduction dimension, so K/V
// values are formed before the dot); [PR113] "feat(kvcache): 8-bit DSV4
// window/compressed KV behind --kv-cache-dtype" §Testing (split-k decode,
// masked (-1) columns).
//
// Work item = (sequence b, chunk of item_pages pages, kv head, group of GT
// query heads).  Items are enumerated on the device from seq_lens (an
// exclusive scan in LDS); a persistent grid strides over them.
//
// Inside an item each of the 4 waves streams its own pages (page groups of
// PPS pages dealt round-robin), with the next groups' K and V codes and
// scales loaded into registers while the current group is computed, and no
// block barrier in the loop:
//   - a lane owns EPL consecutive elements of a token row (one 16-byte load);
//     its partial q.k over that slice is multiplied by the K block scale in
//     fp32 (the code sum itself is exact) and summed over the LPT lanes of
//     the row, giving log2-domain scores in registers;
//   - softmax weights against a reference fixed per item and head (the
//     largest score of the wave's first step; see the stream loop);
//   - p * s_v per (row, head) weights the V codes into fp32 accumulators
//     (for e4m3 codes two rows at a time, as bf16 pairs in dot2 products).
// Rows past the sequence end and masked pages are never multiplied, so NaN
// codes or scales in unused slots cannot reach the output.  The four waves
// are merged through LDS at the end of the item.  A sequence that fits one
// item writes its output directly; otherwise each item writes (m, l, acc)
// to the workspace and the last workgroup to finish a (sequence, kv head,
// head group) -- found with a counter that it resets -- merges them.
#include "kvq_attn.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kWaves = kDecodeWaves;
// Register buffers per wave: the loads of a step are issued kDepth steps
// before it is computed.
constexpr int kDepth = kGqaDepth;
constexpr int kThreads = 64 * kWaves;

template <int QT, int D>
struct Geo {
  static constexpr int ESZ = gqa_elem_bytes(QT);                         // bytes per element
  static constexpr int EPL = (QT == QT_BF16) ? 8 : (D >= 64 ? 16 : 8);   // elements per lane
  static constexpr int NDW = EPL * ESZ / 4;                              // dwords per lane load
  static constexpr int LPT = D / EPL;                                    // lanes per token row
  static constexpr int TPL = 64 / LPT;                                   // rows per wave load
  static constexpr int LPP = kPageSize / TPL;                            // loads per page
  static constexpr int NB = D / 32;                                      // scales per row
  static constexpr int PPS = gqa_pages_per_step(QT, D);                  // pages per step
  static constexpr int ROWS = PPS * LPP;                                 // rows per lane per step
  static_assert(LPT >= 2 && LPT <= 64 && (LPT & (LPT - 1)) == 0, "lane split");
  static_assert(TPL <= kPageSize, "a wave load must stay inside one page");
};

struct GqaParams {
  DecodeArgs a;
  int gt, n_hg;
  ItemRule rule;     // work item size (see plan_items)
  int fused;         // merge split-K partials in the last workgroup (else a merge kernel)
  float scale_log2;  // sm_scale * log2(e)
  int* prefix;       // [batch + 1] items before each sequence (written by block 0)
  int* count;        // [batch * units] arrival counters, zero between calls
  float* part_ml;    // [items][gt][2]
  float* part_acc;   // [items][gt][head_dim]
};

template <int NDW>
struct Raw {
  uint32_t w[NDW];
};

template <int NDW>
__device__ __forceinline__ Raw<NDW> load_raw(const uint8_t* p) {
  Raw<NDW> r;
  if constexpr (NDW == 4) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  } else {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    r.w[0] = v.x; r.w[1] = v.y;
  }
  return r;
}

template <int QT, int NDW>
__device__ __forceinline__ void decode_raw(const Raw<NDW>& r, float* o) {
  constexpr int PER = (QT == QT_BF16) ? 2 : 4;
#pragma unroll
  for (int i = 0; i < NDW; ++i) decode_dword<QT>(r.w[i], o + PER * i);
}

template <int NDW>
__device__ __forceinline__ Raw<NDW> buf_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  Raw<NDW> o;
  if constexpr (NDW == 4) {
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal));
    o.w[0] = v.x; o.w[1] = v.y; o.w[2] = v.z; o.w[3] = v.w;
  } else {
    const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNonTemporal));
    o.w[0] = v.x; o.w[1] = v.y;
  }
  return o;
}

// The new token of a decode with append, as one wave meets it.
template <int NDW>
struct NewRow {
  int step, row;  // the wave's step and row index holding the token (step -1: none)
  bool on;        // this lane holds a piece of that row
  Raw<NDW> k, v;  // the piece's codes (bf16 for a bf16 pool)
  float ks, vs;   // its block scales (1 for the types without one)
  int64_t dst;    // the pool row this lane writes after the stream (-1: none)
  uint16_t sk, sv;
};

// Wave-uniform description of one work item.
struct Item {
  int item, b, u, kvh, hg, nc, t0, nt, np, h0, nsteps;
};

template <int PPS, int GT>
__device__ __forceinline__ Item describe(const GqaParams& p, int item_tokens, int item, int b,
                                         int rem, int L, int wave, int units, int G) {
  Item it;
  it.item = item;
  it.b = b;
  const int chunk = rem / units;
  it.u = rem - chunk * units;
  it.kvh = it.u / p.n_hg;
  const int hg = it.u - it.kvh * p.n_hg;
  it.hg = hg;
  it.nc = (L + item_tokens - 1) / item_tokens;
  it.t0 = chunk * item_tokens;
  it.nt = min(item_tokens, L - it.t0);
  it.np = (it.nt + kPageSize - 1) / kPageSize;
  it.h0 = it.kvh * G + hg * GT;
  const int ngroups = (it.np + PPS - 1) / PPS;
  const int steps = (ngroups > wave) ? (ngroups - wave + kWaves - 1) / kWaves : 0;
  // the step loop is unrolled by kDepth and runs at least kDepth steps (a
  // wave with no pages streams masked steps), so every path through it
  // issues the same loads
  it.nsteps = max((steps + kDepth - 1) / kDepth * kDepth, kDepth);
  return it;
}

// One level of a reduce-scatter over lane pairs that differ in lane bit B:
// of the N values a lane holds, it keeps the first half (bit B clear) or the
// second half (bit B set), each summed with the partner lane's copy.  Bits 5
// and 4 pair rows through the gfx950 permlane swaps (the pair they return
// holds, in every lane, its kept value and the partner's); bit 3 pairs
// lanes 8 apart inside a row of 16 through a DPP rotation.
template <int B, int N>
__device__ __forceinline__ void reduce_scatter_level(float* x) {
  constexpr int H = N / 2;
  static_assert(N % 2 == 0 && B >= 3 && B <= 5, "reduce-scatter level");
  if constexpr (B == 5) {
#pragma unroll
    for (int i = 0; i < H; ++i) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[i]), __float_as_uint(x[i + H]),
                                                      false, false);
      x[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
  } else if constexpr (B == 4) {
#pragma unroll
    for (int i = 0; i < H; ++i) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[i]), __float_as_uint(x[i + H]),
                                                      false, false);
      x[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
  } else {
    const bool hi = (threadIdx.x & 8) != 0;
#pragma unroll
    for (int i = 0; i < H; ++i) {
      const float send = hi ? x[i] : x[i + H], keep = hi ? x[i + H] : x[i];
      x[i] = keep + dpp<kRowRor<8>>(send);
    }
  }
}

// The last workgroup of a split sequence merges up to this many chunks per
// thread straight from global memory.
constexpr int kSmallMerge = 16;

// APP: decode with append.  The item that holds a sequence's new token
// (position length - 1) quantizes the token's K and V rows with the store's
// own routine (quantize_piece); the wave whose page group holds the token
// writes its codes and scales to the pools (items of head group 0 only) and
// uses the same codes in place of whatever its load of that slot returned,
// so the result never depends on the order of that store and that load.
template <int QT, int D, int GT, bool APP>
__global__ __launch_bounds__(kThreads) void gqa_decode_kernel(GqaParams p) {
  using Gm = Geo<QT, D>;
  constexpr int EPL = Gm::EPL, LPT = Gm::LPT, TPL = Gm::TPL, LPP = Gm::LPP, NDW = Gm::NDW;
  constexpr int PPS = Gm::PPS, ROWS = Gm::ROWS, NB = Gm::NB, ESZ = Gm::ESZ;
  constexpr int CODE = gqa_code_bytes(QT, D), SCL = gqa_scale_bytes(QT, D);
  // cross-wave partial sums [kWaves][GT][D] at the end of an item, or the
  // merge's chunk weights and sums [2][chunks][GT]
  constexpr int kRed = (kWaves * GT * D > 2 * kMergeMaxWeights) ? kWaves * GT * D : 2 * kMergeMaxWeights;
  extern __shared__ int s_prefix[];  // [batch + 1]
  __shared__ __attribute__((aligned(16))) float s_red[kRed];
  __shared__ float s_ml[kWaves][GT][2];
  __shared__ float s_hm[GT][2];
  __shared__ int s_wave[kWaves];
  __shared__ int s_last;
  // per-wave staging of a step's K and V scales
  __shared__ __attribute__((aligned(16))) uint8_t s_scl[kWaves][(qt_scaled(QT) ? 2 * PPS * SCL : 1)];

  const DecodeArgs& a = p.a;
  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform (an SGPR): page descriptors built from it stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int seg = lane % LPT, tsub = lane / LPT;
  const int d0 = seg * EPL;
  const int units = a.n_kv_heads * p.n_hg;
  const int G = a.n_q_heads / a.n_kv_heads;

  // page ids of the wave's pages of an item: lane s*PPS+k holds step s, page
  // k (-1: masked or past the item).  The load is issued on every lane (the
  // column clamped into the row), so it can be issued speculatively.
  auto load_pids = [&](const Item& it) {
    const int st = lane / PPS, k = lane - st * PPS;
    const int pi = (wave + st * kWaves) * PPS + k;
    const int col = min(it.t0 / kPageSize + pi, a.max_pages - 1);
    // the lane condition is folded into the value through a mask the
    // compiler cannot see into, so the load is not moved under it
    int keep = (lane < it.nsteps * PPS && pi < it.np) ? 0 : -1;
    asm volatile("" : "+v"(keep));
    const int v = a.page_table[(int64_t)it.b * a.pt_stride + col] | keep;
    return (v >= 0 && (int64_t)v < a.num_pages) ? v : -1;
  };
  // the query slice of this lane as bf16 pairs (exact; the softmax scale is
  // applied to each score in fp32)
  uint32_t qb[GT][EPL / 2];
  auto load_q = [&](const Item& it) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      const uint16_t* qrow = a.q + ((int64_t)it.b * a.n_q_heads + it.h0 + h) * D + d0;
#pragma unroll
      for (int e = 0; e < EPL; e += 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(qrow + e);
        qb[h][e / 2 + 0] = v.x;
        qb[h][e / 2 + 1] = v.y;
        qb[h][e / 2 + 2] = v.z;
        qb[h][e / 2 + 3] = v.w;
      }
    }
  };

  // the new token's K and V slices of this lane (bf16 pairs), loaded beside
  // the query of every item (decode with append)
  uint32_t nrow[2][EPL / 2];
  auto load_new = [&](const Item& it) {
    if constexpr (APP) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint16_t* src = a.new_kv[t] + (int64_t)it.b * a.new_stride + it.kvh * D + d0;
#pragma unroll
        for (int e = 0; e < EPL; e += 8) {
          const uint4 v = *reinterpret_cast<const uint4*>(src + e);
          nrow[t][e / 2 + 0] = v.x;
          nrow[t][e / 2 + 1] = v.y;
          nrow[t][e / 2 + 2] = v.z;
          nrow[t][e / 2 + 3] = v.w;
        }
      }
    }
  };

  // The work list.  Up to 64 sequences, every wave builds it alone (lane b
  // holds the items before sequence b, and its length): one load, no LDS,
  // no barrier.  Beside that load, the page ids and query of this
  // workgroup's first item are loaded as if every sequence filled its
  // page-table row; they are used when the actual list gives the same item
  // (the loads are unconditional and in bounds either way).  Larger batches
  // scan seq_lens in LDS.
  const bool small = a.batch <= 64 && (int64_t)a.batch * a.max_pages < (1 << 30);
  int item_tokens, total, wpfx = 0, wlen = 0, pid_spec = -1, raw_len = 0;
  Item spec;
  spec.b = -1;
  if (small) {
    raw_len = a.seq_lens[min(lane, a.batch - 1)];
    const int full = a.max_pages * kPageSize;
    const int g_tokens = rule_item_tokens(p.rule, (int64_t)a.batch * a.max_pages, units);
    const int g_per_seq = (full + g_tokens - 1) / g_tokens * units;
    const int g_item = min((int)blockIdx.x, a.batch * g_per_seq - 1);
    const int g_b = g_item / g_per_seq;
    spec = describe<PPS, GT>(p, g_tokens, g_item, g_b, g_item - g_b * g_per_seq, full, wave, units, G);
    pid_spec = load_pids(spec);
    load_q(spec);
    load_new(spec);
    // the length is first used here, after the speculative loads are issued
    __builtin_amdgcn_sched_barrier(0);
    wlen = lane < a.batch ? min(max(raw_len, 0), a.max_pages * kPageSize) : 0;
    item_tokens = plan_items_wave(p.rule, units, wlen, &wpfx, &total);
    if ((int)blockIdx.x >= a.batch * g_per_seq) spec.b = -1;
  } else {
    item_tokens = plan_items<kThreads>(a, p.rule, units, s_prefix, s_wave);
    total = s_prefix[a.batch];
  }
  // items before sequence b (b <= batch), uniform b
  auto prefix_of = [&](int b) {
    if (!small) return s_prefix[b];
    return b < a.batch ? __builtin_amdgcn_readlane(wpfx, b) : total;
  };
  if (blockIdx.x == 0) {
    if (small) {
      if (wave == 0 && lane < a.batch) p.prefix[lane] = wpfx;
      if (tid == 0) p.prefix[a.batch] = total;
    } else {
      for (int b = tid; b <= a.batch; b += kThreads) p.prefix[b] = s_prefix[b];
    }
  }
  // a sequence with no valid length has no items: its output is 0, lse -inf
  for (int b = blockIdx.x; b < a.batch; b += gridDim.x) {
    if (prefix_of(b) != prefix_of(b + 1)) continue;
    for (int i = tid; i < a.n_q_heads * D; i += kThreads)
      a.out[(int64_t)b * a.n_q_heads * D + i] = 0;
    if (a.lse)
      for (int h = tid; h < a.n_q_heads; h += kThreads) a.lse[(int64_t)b * a.n_q_heads + h] = -INFINITY;
  }
  if ((int)blockIdx.x >= total) return;  // uniform over the block

  // per-lane offsets inside a (page, kv head) chunk, the same for every page
  uint32_t code_off[LPP], scale_off[LPP];
#pragma unroll
  for (int i = 0; i < LPP; ++i) {
    code_off[i] = (uint32_t)(((i * TPL + tsub) * D + d0) * ESZ);
    scale_off[i] = (uint32_t)(((i * TPL + tsub) * NB + (d0 >> 5)) * 2);
  }
  const int64_t page_rows = (int64_t)a.n_kv_heads * kPageSize;

  // A step's loads.  The scales of a (page, kv head) chunk (SCL bytes) come
  // in one 4-byte-per-lane load: lane L holds bytes [4L, 4L+4), lanes past
  // the chunk read 0 through the descriptor's bound.  They are staged through
  // a wave-private LDS area when the step is computed.
  struct Buf {
    Raw<NDW> k[ROWS], v[ROWS];
    uint32_t ks[PPS], vs[PPS];
  };
  // Loads of one step.  They are issued on every path, never under a
  // branch: the hardware counts outstanding loads in issue order, and a load
  // skipped on one path would make the compiler wait for every load in
  // flight (the prefetch included) before the next compute.  A masked page
  // or a step past the end (valid == false) gets zero-length descriptors,
  // whose loads return 0 without touching memory; such rows are never
  // used.  The page base is wave-uniform; lanes add 32-bit
  // offsets; the descriptor bounds each access to its page chunk.
  auto load_step = [&](const Item& it, int pid, int st, bool valid, Buf& X) {
#pragma unroll
    for (int k = 0; k < PPS; ++k) {
      const int Pr = __builtin_amdgcn_readlane(pid, min(st * PPS + k, 63));
      const bool live = valid && Pr >= 0;
      const int64_t row0 = (int64_t)max(Pr, 0) * page_rows + (int64_t)it.kvh * kPageSize;
      const auto rk = page_rsrc(a.k_pool + row0 * D * ESZ, live ? CODE : 0);
      const auto rv = page_rsrc(a.v_pool + row0 * D * ESZ, live ? CODE : 0);
#pragma unroll
      for (int i = 0; i < LPP; ++i) {
        X.k[k * LPP + i] = buf_load<NDW>(rk, code_off[i]);
        X.v[k * LPP + i] = buf_load<NDW>(rv, code_off[i]);
      }
      if constexpr (qt_scaled(QT)) {
        const auto rks = page_rsrc(a.k_scales + row0 * NB, live ? SCL : 0);
        const auto rvs = page_rsrc(a.v_scales + row0 * NB, live ? SCL : 0);
        X.ks[k] = __builtin_amdgcn_raw_buffer_load_b32(rks, lane * 4, 0, 0);
        X.vs[k] = __builtin_amdgcn_raw_buffer_load_b32(rvs, lane * 4, 0, 0);
      }
    }
  };

  float mref[GT], smax[GT], lsum[GT], acc[GT][EPL];

  // Log2-domain scores of a step's rows (-inf for rows on a masked page or
  // past the item end), their validity and the V scale of each row.
  auto scores = [&](const Item& it, int pid, int st, Buf& X, float (*sc)[GT], bool* ok,
                    float* vsf, const NewRow<NDW>& nr) {
    // scales of this step's pages -> this wave's LDS area -> one per row
    float ksf[ROWS];
    if constexpr (qt_scaled(QT)) {
      uint8_t* sw = s_scl[wave];
#pragma unroll
      for (int k = 0; k < PPS; ++k) {
        if (lane * 4 < SCL) {
          *reinterpret_cast<uint32_t*>(sw + (2 * k) * SCL + lane * 4) = X.ks[k];
          *reinterpret_cast<uint32_t*>(sw + (2 * k + 1) * SCL + lane * 4) = X.vs[k];
        }
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int k = 0; k < PPS; ++k)
#pragma unroll
        for (int i = 0; i < LPP; ++i) {
          ksf[k * LPP + i] = f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(sw + (2 * k) * SCL + scale_off[i]));
          vsf[k * LPP + i] = f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(sw + (2 * k + 1) * SCL + scale_off[i]));
        }
      __builtin_amdgcn_wave_barrier();
    } else {
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        ksf[r] = 1.0f;
        vsf[r] = 1.0f;
      }
    }
    // the new token's row (decode with append): its codes and scales replace
    // what the load of its slot returned
    if constexpr (APP) {
      if (st == nr.step) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
          if (r == nr.row && nr.on) {
            X.k[r] = nr.k;
            X.v[r] = nr.v;
            ksf[r] = nr.ks;
            vsf[r] = nr.vs;
          }
      }
    }
    // row validity: page present and token before the item end (a select,
    // not a branch, so the step's work stays one scheduling region)
#pragma unroll
    for (int k = 0; k < PPS; ++k) {
      const int P = __builtin_amdgcn_readlane(pid, min(st * PPS + k, 63));
      const int pi = (wave + st * kWaves) * PPS + k;
      const int lim = P >= 0 ? it.nt : 0;
#pragma unroll
      for (int i = 0; i < LPP; ++i) ok[k * LPP + i] = pi * kPageSize + i * TPL + tsub < lim;
    }
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      uint32_t kb2[EPL / 2];  // codes as bf16 pairs (exact)
#pragma unroll
      for (int i = 0; i < NDW; ++i)
        decode_dword_bf16x2<QT>(X.k[r].w[i], kb2 + i * (QT == QT_BF16 ? 1 : 2));
      const float f = ksf[r] * p.scale_log2;
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        float t = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL / 2; ++e) t = dot2_bf16(qb[h][e], kb2[e], t);
        sc[r][h] = t * f;
      }
    }
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        const float t = group_sum<LPT>(sc[r][h]);
        sc[r][h] = ok[r] ? t : -INFINITY;
      }
  };

  // Weights against the fixed reference and the weighted sum of V.  Codes
  // of invalid rows are zeroed (their weight is 0, but the slot may hold NaN
  // codes or scales).
  auto accumulate = [&](const Buf& X, float (*sc)[GT], const bool* ok, const float* vsf) {
    float w[ROWS][GT];
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        smax[h] = fmaxf(smax[h], sc[r][h]);
        const float pr = __builtin_amdgcn_exp2f(sc[r][h] - mref[h]);  // 0 for -inf
        lsum[h] += pr;
        w[r][h] = ok[r] ? pr * vsf[r] : 0.0f;
      }
    if constexpr (qt_f8(QT) && ROWS % 2 == 0) {
      // two rows at a time: each element's two codes form one bf16 pair
      // (exact) and meet the two rows' weights (rounded to bf16) in a dot2
#pragma unroll
      for (int r = 0; r < ROWS; r += 2) {
        const uint32_t k0 = ok[r] ? 0xffffffffu : 0u, k1 = ok[r + 1] ? 0xffffffffu : 0u;
        uint32_t wp[GT];
#pragma unroll
        for (int h = 0; h < GT; ++h) wp[h] = pack_bf16x2(w[r][h], w[r + 1][h]);
#pragma unroll
        for (int i = 0; i < NDW; ++i) {
          const uint32_t a = X.v[r].w[i] & k0, b = X.v[r + 1].w[i] & k1;
          const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x05010400u);  // a0 b0 a1 b1
          const uint32_t hi = __builtin_amdgcn_perm(b, a, 0x07030602u);  // a2 b2 a3 b3
          uint32_t vp[4];
          decode_dword_bf16x2<QT>(lo, vp);
          decode_dword_bf16x2<QT>(hi, vp + 2);
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int h = 0; h < GT; ++h) acc[h][4 * i + j] = dot2_bf16(vp[j], wp[h], acc[h][4 * i + j]);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const uint32_t keep = ok[r] ? 0xffffffffu : 0u;
        Raw<NDW> vr;
#pragma unroll
        for (int i = 0; i < NDW; ++i) vr.w[i] = X.v[r].w[i] & keep;
        float vv[EPL];
        decode_raw<QT, NDW>(vr, vv);
#pragma unroll
        for (int h = 0; h < GT; ++h)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(w[r][h], vv[e], acc[h][e]);
      }
    }
  };

  Buf R[kDepth];
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    int bq;
    if (small) {
      bq = wave_item_seq(wpfx, a.batch, item);
    } else {
      int lo = 0, hi = a.batch - 1;
      while (lo < hi) {  // largest b with s_prefix[b] <= item
        const int mid = (lo + hi + 1) >> 1;
        if (s_prefix[mid] <= item) lo = mid; else hi = mid - 1;
      }
      bq = lo;
    }
    const int L = small ? __builtin_amdgcn_readlane(wlen, bq) : clamped_len(a, bq);
    const Item cur = describe<PPS, GT>(p, item_tokens, item, bq, item - prefix_of(bq), L, wave, units, G);
    const bool hit = cur.b == spec.b && cur.u == spec.u && cur.t0 == spec.t0 && cur.nt == spec.nt;
    spec.b = -1;  // the speculative loads serve the first item only
    int pid_cur = pid_spec;
    if (!hit) {
      pid_cur = load_pids(cur);
      load_q(cur);
      load_new(cur);
    }
    // The new token (decode with append), if this item holds it: the step
    // and row index where this wave meets it, and its codes and scales.
    NewRow<NDW> nr;
    nr.step = -1;
    nr.dst = -1;
    if constexpr (APP) {
      const int raw = small ? __builtin_amdgcn_readlane(raw_len, bq) : a.seq_lens[bq];
      const int tn = raw - 1;
      if (raw >= 1 && raw <= a.max_pages * kPageSize && tn >= cur.t0 && tn < cur.t0 + cur.nt) {
        const int pi = (tn - cur.t0) / kPageSize, grp = pi / PPS;
        if (grp % kWaves == wave) {  // uniform: the wave that streams its page
          const int st = grp / kWaves, k = pi - grp * PPS, r = tn % kPageSize;
          nr.step = st;
          nr.row = k * LPP + r / TPL;
          nr.on = tsub == r % TPL;
          uint16_t sb[2];
          quantize_piece<QT, EPL>(nrow[0], nr.k.w, &sb[0]);
          quantize_piece<QT, EPL>(nrow[1], nr.v.w, &sb[1]);
          nr.ks = qt_scaled(QT) ? f16_bits_to_f32(sb[0]) : 1.0f;
          nr.vs = qt_scaled(QT) ? f16_bits_to_f32(sb[1]) : 1.0f;
          const int P = __builtin_amdgcn_readlane(pid_cur, st * PPS + k);
          if (P >= 0 && cur.hg == 0 && nr.on)
            nr.dst = ((int64_t)P * a.n_kv_heads + cur.kvh) * kPageSize + r;
          nr.sk = sb[0];
          nr.sv = sb[1];
        }
      }
    }
    // Stream the item's steps, kDepth steps' loads in flight (cur.nsteps is
    // a multiple of kDepth).  The softmax reference of each head stays fixed
    // over a pass: the largest score of the wave's first step (0 when it has
    // none), so the weights 2^(s - mref) need no running-max update, no
    // cross-lane reduction and no rescaling.  A pass whose largest score ends
    // more than 2^64 away from the reference (weights could overflow, or all
    // underflow) is streamed again with that score as the reference.
    float M[GT];  // largest score per head over the wave's rows of the item
    for (int pass = 0;; ++pass) {
#pragma unroll
      for (int k = 0; k < kDepth; ++k) load_step(cur, pid_cur, k, k < cur.nsteps, R[k]);
      if (pass == 0) {
        float sc0[ROWS][GT], vs0[ROWS];
        bool ok0[ROWS];
        scores(cur, pid_cur, 0, R[0], sc0, ok0, vs0, nr);
#pragma unroll
        for (int h = 0; h < GT; ++h) {
          float t = sc0[0][h];
#pragma unroll
          for (int r = 1; r < ROWS; ++r) t = fmaxf(t, sc0[r][h]);
          t = stride_max<LPT>(t);
          mref[h] = (t == -INFINITY) ? 0.0f : t;
        }
      }
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        smax[h] = -INFINITY;
        lsum[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;
      }
      for (int st = 0; st < cur.nsteps; st += kDepth) {
#pragma unroll
        for (int k = 0; k < kDepth; ++k) {
          float sc[ROWS][GT], vsf[ROWS];
          bool ok[ROWS];
          scores(cur, pid_cur, st + k, R[k], sc, ok, vsf, nr);
          accumulate(R[k], sc, ok, vsf);
          const int sn = st + k + kDepth;
          load_step(cur, pid_cur, sn, sn < cur.nsteps, R[k]);
        }
      }
      bool redo = false;
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        M[h] = stride_max<LPT>(smax[h]);
        redo |= M[h] != -INFINITY && (M[h] > mref[h] + 64.0f || M[h] < mref[h] - 64.0f);
      }
      if (!__builtin_amdgcn_ballot_w64(redo)) break;
#pragma unroll
      for (int h = 0; h < GT; ++h) mref[h] = (M[h] == -INFINITY) ? 0.0f : M[h];
    }
    // the new row goes to the pool after the stream (its codes were used from
    // registers): stores issued earlier would sit in the load counter ahead
    // of the stream's first steps
    if constexpr (APP) {
      if (nr.dst >= 0) {
        const int64_t row = nr.dst;
        uint8_t* kp = const_cast<uint8_t*>(a.k_pool) + (row * D + d0) * ESZ;
        uint8_t* vp = const_cast<uint8_t*>(a.v_pool) + (row * D + d0) * ESZ;
        if constexpr (NDW == 4) {
          *reinterpret_cast<uint4*>(kp) = make_uint4(nr.k.w[0], nr.k.w[1], nr.k.w[2], nr.k.w[3]);
          *reinterpret_cast<uint4*>(vp) = make_uint4(nr.v.w[0], nr.v.w[1], nr.v.w[2], nr.v.w[3]);
        } else {
          *reinterpret_cast<uint2*>(kp) = make_uint2(nr.k.w[0], nr.k.w[1]);
          *reinterpret_cast<uint2*>(vp) = make_uint2(nr.v.w[0], nr.v.w[1]);
        }
        if constexpr (qt_scaled(QT)) {
          if ((seg & (32 / EPL - 1)) == 0) {
            const_cast<uint16_t*>(a.k_scales)[row * NB + (d0 >> 5)] = nr.sk;
            const_cast<uint16_t*>(a.v_scales)[row * NB + (d0 >> 5)] = nr.sv;
          }
        }
      }
    }
    // a head with no valid row here contributes nothing to the merges
    float m[GT];
#pragma unroll
    for (int h = 0; h < GT; ++h) m[h] = (M[h] == -INFINITY) ? -INFINITY : mref[h];

    // ---- merge the rows held by other lanes, then the four waves ------------------
    // Row sums over the TPL lanes of a column slice; the accumulators by a
    // reduce-scatter when those lanes differ in lane bits 3..5 (LPT >= 8):
    // lane (tsub, seg) ends with NK consecutive values of its slice, the
    // sums of X[tsub * NK ..] over the TPL lanes, X[h * EPL + e] = acc[h][e].
    constexpr int NX = GT * EPL;
    constexpr bool kScatter = LPT >= 8;
    constexpr int NK = kScatter ? NX / TPL : NX;
    float xs[NX];
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      lsum[h] = stride_sum<LPT>(lsum[h]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) xs[h * EPL + e] = acc[h][e];
    }
    if constexpr (kScatter) {
      reduce_scatter_level<5, NX>(xs);
      if constexpr (LPT <= 16) reduce_scatter_level<4, NX / 2>(xs);
      if constexpr (LPT <= 8) reduce_scatter_level<3, NX / 4>(xs);
    } else {
#pragma unroll
      for (int j = 0; j < NX; ++j) xs[j] = stride_sum<LPT>(xs[j]);
    }
    __syncthreads();  // s_red / s_ml of the previous item are free
    if (kScatter || tsub == 0) {
      const int j0 = kScatter ? tsub * NK : 0;
#pragma unroll
      for (int i = 0; i < NK; i += (NK % 4 == 0 ? 4 : 1)) {
        const int j = j0 + i, h = j / EPL, e = j - h * EPL;
        float* dst = &s_red[(wave * GT + h) * D + d0 + e];
        if constexpr (NK % 4 == 0)
          *reinterpret_cast<f32x4*>(dst) = f32x4{xs[i], xs[i + 1], xs[i + 2], xs[i + 3]};
        else
          *dst = xs[i];
      }
    }
    if (lane == 0)
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        s_ml[wave][h][0] = m[h];
        s_ml[wave][h][1] = lsum[h];
      }
    __syncthreads();
    // every thread weighs the four waves itself: M = max m_w, weights
    // 2^(m_w - M) (LDS broadcast reads; no further barrier)
    const int b = cur.b, u = cur.u, nc = cur.nc, h0 = cur.h0;
    for (int idx = tid; idx < GT * D; idx += kThreads) {
      const int h = idx / D, d = idx - h * D;
      float mw[kWaves], M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        mw[w] = s_ml[w][h][0];
        M = fmaxf(M, mw[w]);
      }
      float v = 0.0f, Ls = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float wt = exp2_rel(mw[w], M);
        v += wt * s_red[(w * GT + h) * D + d];
        Ls += wt * s_ml[w][h][1];
      }
      if (nc == 1) {
        const int64_t orow = (int64_t)b * a.n_q_heads + h0 + h;
        a.out[orow * D + d] = (uint16_t)bf16_rne(Ls > 0.0f ? v / Ls : 0.0f);
        if (d == 0 && a.lse) a.lse[orow] = (M == -INFINITY) ? -INFINITY : (M + log2f(Ls)) * kLn2;
      } else {
        store_agent(&p.part_acc[((int64_t)item * GT + h) * D + d], v);
        if (d == 0) {
          store_agent(&p.part_ml[((int64_t)item * GT + h) * 2 + 0], M);
          store_agent(&p.part_ml[((int64_t)item * GT + h) * 2 + 1], Ls);
        }
      }
    }

    if (nc > 1 && p.fused) {
      // ---- the last item of this (sequence, kv head, head group) merges -------------
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
        const int first = prefix_of(b) + u;  // item of chunk c: first + c * units
        const int64_t cstride = (int64_t)units * GT * D;  // between chunks of this group
        if (nc <= kSmallMerge) {
          // Each thread merges its own columns from global memory: the
          // chunks' partial sums and (m, l) are loaded together, then
          // M = max m_c, weights 2^(m_c - M).  No LDS, no barrier.
          for (int idx = tid; idx < GT * D; idx += kThreads) {
            const int h = idx / D, d = idx - h * D;
            const float* src = p.part_acc + ((int64_t)first * GT + h) * D + d;
            const float* ml = p.part_ml + ((int64_t)first * GT + h) * 2;
            float x[kSmallMerge], mc[kSmallMerge], lc[kSmallMerge];
#pragma unroll
            for (int c = 0; c < kSmallMerge; ++c) {
              x[c] = (c < nc) ? load_agent(src + c * cstride) : 0.0f;
              mc[c] = (c < nc) ? load_agent(ml + c * units * GT * 2) : -INFINITY;
              lc[c] = (c < nc) ? load_agent(ml + c * units * GT * 2 + 1) : 0.0f;
            }
            float M = mc[0];
#pragma unroll
            for (int c = 1; c < kSmallMerge; ++c) M = fmaxf(M, mc[c]);
            float v = 0.0f, Ls = 0.0f;
#pragma unroll
            for (int c = 0; c < kSmallMerge; ++c) {
              const float w = exp2_rel(mc[c], M);
              v += w * x[c];
              Ls += w * lc[c];
            }
            const int64_t orow = (int64_t)b * a.n_q_heads + h0 + h;
            a.out[orow * D + d] = (uint16_t)bf16_rne(Ls > 0.0f ? v / Ls : 0.0f);
            if (d == 0 && a.lse)
              a.lse[orow] = (M == -INFINITY) ? -INFINITY : (M + log2f(Ls)) * kLn2;
          }
        } else {
          // Many chunks: their (m, l) go through LDS, one wave per head
          // forms the weights, then each thread sums its columns.
          float* s_l = s_red + kMergeMaxWeights;
          for (int idx = tid; idx < nc * GT; idx += kThreads) {
            const int c = idx / GT, h = idx - c * GT;
            const float* ml = &p.part_ml[((int64_t)(first + c * units) * GT + h) * 2];
            s_red[idx] = load_agent(ml);
            s_l[idx] = load_agent(ml + 1);
          }
          __syncthreads();
          for (int h = wave; h < GT; h += kWaves) {
            float M = -INFINITY;
            for (int c = lane; c < nc; c += 64) M = fmaxf(M, s_red[c * GT + h]);
            M = stride_max<1>(M);
            float Ls = 0.0f;
            for (int c = lane; c < nc; c += 64) {
              const float w = exp2_rel(s_red[c * GT + h], M);
              Ls += w * s_l[c * GT + h];
              s_red[c * GT + h] = w;
            }
            Ls = stride_sum<1>(Ls);
            if (lane == 0) {
              s_hm[h][0] = M;
              s_hm[h][1] = Ls;
            }
          }
          __syncthreads();
          for (int idx = tid; idx < GT * D; idx += kThreads) {
            const int h = idx / D, d = idx - h * D;
            const float* src = p.part_acc + ((int64_t)first * GT + h) * D + d;
            float v = 0.0f;
            for (int c0 = 0; c0 < nc; c0 += 16) {  // 16 loads in flight per thread
              float x[16];
#pragma unroll
              for (int j = 0; j < 16; ++j)
                x[j] = (c0 + j < nc) ? load_agent(src + (c0 + j) * cstride) : 0.0f;
#pragma unroll
              for (int j = 0; j < 16; ++j)
                if (c0 + j < nc) v += s_red[(c0 + j) * GT + h] * x[j];
            }
            const float M = s_hm[h][0], Ls = s_hm[h][1];
            const int64_t orow = (int64_t)b * a.n_q_heads + h0 + h;
            a.out[orow * D + d] = (uint16_t)bf16_rne(Ls > 0.0f ? v / Ls : 0.0f);
            if (d == 0 && a.lse)
              a.lse[orow] = (M == -INFINITY) ? -INFINITY : (M + log2f(Ls)) * kLn2;
          }
        }
        if (tid == 0)  // ready for the next call
          __hip_atomic_store(&p.count[(int64_t)b * units + u], 0, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

template <int QT, int D, int GT>
hipError_t launch_one(const GqaParams& gp, int grid, hipStream_t s) {
  const size_t dyn = (size_t)(gp.a.batch + 1) * sizeof(int);
  if (gp.a.new_kv[0])
    gqa_decode_kernel<QT, D, GT, true><<<grid, kThreads, dyn, s>>>(gp);
  else
    gqa_decode_kernel<QT, D, GT, false><<<grid, kThreads, dyn, s>>>(gp);
  return hipGetLastError();
}

template <int QT, int D>
hipError_t launch_gt(const GqaParams& gp, int grid, hipStream_t s) {
  switch (gp.gt) {
    case 1: return launch_one<QT, D, 1>(gp, grid, s);
    case 2: return launch_one<QT, D, 2>(gp, grid, s);
    case 4: return launch_one<QT, D, 4>(gp, grid, s);
    default: return launch_one<QT, D, 8>(gp, grid, s);
  }
}

template <int QT>
hipError_t launch_d(const GqaParams& gp, int grid, hipStream_t s) {
  switch (gp.a.head_dim_qk) {
    case 32: return launch_gt<QT, 32>(gp, grid, s);
    case 64: return launch_gt<QT, 64>(gp, grid, s);
    case 128: return launch_gt<QT, 128>(gp, grid, s);
    default: return launch_gt<QT, 256>(gp, grid, s);
  }
}

template <int QT>
hipError_t launch_typed(const DecodeArgs& a, const DecodePlan& plan, int num_cus, hipStream_t s) {
  char* ws = static_cast<char*>(a.workspace);
  GqaParams gp;
  gp.a = a;
  gp.gt = plan.gt;
  gp.n_hg = plan.n_hg;
  gp.rule = ItemRule{plan.step, plan.min_pages, plan.cap_pages, plan.target};
  gp.fused = plan.fused_merge ? 1 : 0;
  gp.scale_log2 = a.sm_scale * kLog2e;
  gp.prefix = reinterpret_cast<int*>(ws + plan.off_prefix);
  gp.count = reinterpret_cast<int*>(ws + plan.off_count);
  gp.part_ml = reinterpret_cast<float*>(ws + plan.off_ml);
  gp.part_acc = reinterpret_cast<float*>(ws + plan.off_acc);
  // Items are sized for about one per compute unit (plan.target); the grid
  // holds two workgroups per compute unit.  When the items are that few, the
  // second half finds no item and exits after the prologue, so each compute
  // unit streams one item alone; when there are many more items (long or
  // many sequences), the persistent grid strides over them with two
  // workgroups per compute unit, one streaming while the other is between
  // items.
  int64_t grid = 2 * (int64_t)num_cus;
  if (grid > plan.max_items) grid = plan.max_items;
  if (a.items_hint > 0 && grid > a.items_hint) grid = a.items_hint;  // exact from host lengths
  if (grid < 1) grid = 1;
  const hipError_t e = launch_d<QT>(gp, (int)grid, s);
  if (e != hipSuccess || plan.fused_merge) return e;
  return launch_gqa_merge(a, plan, s);
}

}  // namespace

// The library's build compiles this file once per storage type
// (-DKVQ_DECODE_QT); compiled alone it defines all five.
#define KVQ_DEFINE_TYPED(QT)                                                                  \
  template <>                                                                                \
  hipError_t launch_gqa_decode_typed<QT>(const DecodeArgs& a, const DecodePlan& plan,        \
                                         int num_cus, hipStream_t s) {                       \
    return launch_typed<QT>(a, plan, num_cus, s);                                            \
  }
#ifdef KVQ_DECODE_QT
KVQ_DEFINE_TYPED(KVQ_DECODE_QT)
#else
KVQ_DEFINE_TYPED(QT_BF16)
KVQ_DEFINE_TYPED(QT_FP8)
KVQ_DEFINE_TYPED(QT_Q8)
KVQ_DEFINE_TYPED(QT_FP8C)
KVQ_DEFINE_TYPED(QT_BF8C)
#endif

}  // namespace kvq
