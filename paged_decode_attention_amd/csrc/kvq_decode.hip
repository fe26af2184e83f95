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
// PPS pages dealt round-robin), with the next group's K and V codes and
// scales loaded into registers while the current group is computed, so a
// wave keeps about 8.5 KB in flight and no block barrier sits in the loop:
//   - a lane owns EPL consecutive elements of a token row (one 16-byte load);
//     its partial q.k over that slice is multiplied by the K block scale in
//     fp32 (the code sum itself is exact) and summed over the LPT lanes of
//     the row, giving log2-domain scores in registers;
//   - an online softmax per head (running max, rescaled only when it grows);
//   - p * s_v per (row, head) weights the V codes into fp32 accumulators.
// Rows past the sequence end and masked pages are never multiplied, so NaN
// codes or scales in unused slots cannot reach the output.  The four waves
// are merged through LDS at the end of the item.  A sequence that fits one
// item writes its output directly; otherwise each item writes (m, l, acc)
// to the workspace and the last workgroup to finish a (sequence, kv head,
// head group) -- found with a counter that it resets -- merges them.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

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
  int gt, n_hg, item_tokens;
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

// Sum over aligned groups of W consecutive lanes.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = 1; m < W; m <<= 1) v += shfl_xor_f(v, m);
  return v;
}
// Sum / max over the lanes l, l^S, l^2S, ... (all lanes with equal l mod S).
template <int S>
__device__ __forceinline__ float stride_sum(float v) {
#pragma unroll
  for (int m = S; m < 64; m <<= 1) v += shfl_xor_f(v, m);
  return v;
}
template <int S>
__device__ __forceinline__ float stride_max(float v) {
#pragma unroll
  for (int m = S; m < 64; m <<= 1) v = fmaxf(v, shfl_xor_f(v, m));
  return v;
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

// exp2(x - m) that is 0 (not NaN) when both are -inf.
__device__ __forceinline__ float exp2_rel(float x, float m) {
  return (x == -INFINITY) ? 0.0f : exp2f(x - m);
}

template <int QT, int D, int GT>
__global__ __launch_bounds__(kThreads) void gqa_decode_kernel(GqaParams p) {
  using Gm = Geo<QT, D>;
  constexpr int EPL = Gm::EPL, LPT = Gm::LPT, TPL = Gm::TPL, LPP = Gm::LPP, NDW = Gm::NDW;
  constexpr int PPS = Gm::PPS, ROWS = Gm::ROWS, NB = Gm::NB, ESZ = Gm::ESZ;
  // cross-wave partial sums [kWaves][GT][D] at the end of an item, or the
  // merge's chunk weights [chunks][GT]
  constexpr int kRed = (kWaves * GT * D > kMergeMaxWeights) ? kWaves * GT * D : kMergeMaxWeights;
  extern __shared__ int s_prefix[];  // [batch + 1]
  __shared__ float s_red[kRed];
  __shared__ float s_ml[kWaves][GT][2];
  __shared__ float s_hm[GT][2];
  __shared__ int s_wave[kWaves];
  __shared__ int s_last;

  const DecodeArgs& a = p.a;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seg = lane % LPT, tsub = lane / LPT;
  const int d0 = seg * EPL;
  const int units = a.n_kv_heads * p.n_hg;
  const int G = a.n_q_heads / a.n_kv_heads;

  build_prefix(a, p.item_tokens, units, s_prefix, s_wave);
  const int total = s_prefix[a.batch];
  if (blockIdx.x == 0)
    for (int b = tid; b <= a.batch; b += kThreads) p.prefix[b] = s_prefix[b];
  // a sequence with no valid length has no items: its output is 0, lse -inf
  for (int b = blockIdx.x; b < a.batch; b += gridDim.x) {
    if (s_prefix[b] != s_prefix[b + 1]) continue;
    for (int i = tid; i < a.n_q_heads * D; i += kThreads)
      a.out[(int64_t)b * a.n_q_heads * D + i] = 0;
    if (a.lse)
      for (int h = tid; h < a.n_q_heads; h += kThreads) a.lse[(int64_t)b * a.n_q_heads + h] = -INFINITY;
  }

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    // ---- which (sequence, chunk, kv head, head group) ----------------------------
    int lo = 0, hi = a.batch - 1;
    while (lo < hi) {  // largest b with s_prefix[b] <= item
      const int mid = (lo + hi + 1) >> 1;
      if (s_prefix[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int rem = item - s_prefix[b];
    const int chunk = rem / units;
    const int u = rem - chunk * units;
    const int kvh = u / p.n_hg;
    const int hg = u - kvh * p.n_hg;
    const int L = clamped_len(a, b);
    const int nc = (L + p.item_tokens - 1) / p.item_tokens;
    const int t0 = chunk * p.item_tokens;
    const int nt = min(p.item_tokens, L - t0);
    const int np = (nt + kPageSize - 1) / kPageSize;
    const int h0 = kvh * G + hg * GT;

    // ---- this wave's pages: steps s = 0..nsteps-1, each PPS pages ----------------
    const int ngroups = (np + PPS - 1) / PPS;
    const int nsteps = (ngroups > wave) ? (ngroups - wave + kWaves - 1) / kWaves : 0;
    int pid_lane = -1;  // lane s*PPS+k holds the page id of step s, page k
    if (lane < nsteps * PPS) {
      const int s = lane / PPS, k = lane - s * PPS;
      const int pi = (wave + s * kWaves) * PPS + k;
      if (pi < np) {
        const int pid = a.page_table[(int64_t)b * a.pt_stride + t0 / kPageSize + pi];
        pid_lane = (pid >= 0 && (int64_t)pid < a.num_pages) ? pid : -1;
      }
    }

    // query slice of this lane, log2 domain
    float qf[GT][EPL];
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      const uint16_t* qrow = a.q + ((int64_t)b * a.n_q_heads + h0 + h) * D + d0;
#pragma unroll
      for (int e = 0; e < EPL; e += 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(qrow + e);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          qf[h][e + 2 * k] = bf16_lo(w[k]) * p.scale_log2;
          qf[h][e + 2 * k + 1] = bf16_hi(w[k]) * p.scale_log2;
        }
      }
    }

    float m[GT], lsum[GT], acc[GT][EPL];
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      m[h] = -INFINITY;
      lsum[h] = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;
    }

    Raw<NDW> kr[ROWS], vr[ROWS], nkr[ROWS], nvr[ROWS];
    float ks[ROWS], vs[ROWS], nks[ROWS], nvs[ROWS];
    auto load_step = [&](int s, Raw<NDW>* K, Raw<NDW>* V, float* KS, float* VS) {
#pragma unroll
      for (int k = 0; k < PPS; ++k) {
        const int P = __builtin_amdgcn_readlane(pid_lane, s * PPS + k);
        if (P >= 0) {
          const int64_t rbase = ((int64_t)P * a.n_kv_heads + kvh) * kPageSize;
#pragma unroll
          for (int i = 0; i < LPP; ++i) {
            const int64_t r = rbase + i * TPL + tsub;
            K[k * LPP + i] = load_raw<NDW>(a.k_pool + (r * D + d0) * ESZ);
            V[k * LPP + i] = load_raw<NDW>(a.v_pool + (r * D + d0) * ESZ);
            if constexpr (QT != QT_BF16) {
              KS[k * LPP + i] = f16_bits_to_f32(a.k_scales[r * NB + (d0 >> 5)]);
              VS[k * LPP + i] = f16_bits_to_f32(a.v_scales[r * NB + (d0 >> 5)]);
            } else {
              KS[k * LPP + i] = 1.0f;
              VS[k * LPP + i] = 1.0f;
            }
          }
        }
      }
    };

    if (nsteps > 0) load_step(0, nkr, nvr, nks, nvs);
    for (int s = 0; s < nsteps; ++s) {
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        kr[r] = nkr[r];
        vr[r] = nvr[r];
        ks[r] = nks[r];
        vs[r] = nvs[r];
      }
      if (s + 1 < nsteps) load_step(s + 1, nkr, nvr, nks, nvs);

      // row validity: page present and token before the sequence end
      bool ok[ROWS];
#pragma unroll
      for (int k = 0; k < PPS; ++k) {
        const int P = __builtin_amdgcn_readlane(pid_lane, s * PPS + k);
        const int pi = (wave + s * kWaves) * PPS + k;
#pragma unroll
        for (int i = 0; i < LPP; ++i)
          ok[k * LPP + i] = (P >= 0) && (pi * kPageSize + i * TPL + tsub < nt);
      }

      // scores
      float sc[ROWS][GT];
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        float kv[EPL];
        decode_raw<QT, NDW>(kr[r], kv);
#pragma unroll
        for (int h = 0; h < GT; ++h) {
          float t = 0.0f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) t = fmaf(qf[h][e], kv[e], t);
          sc[r][h] = t * ks[r];
        }
      }
#pragma unroll
      for (int r = 0; r < ROWS; ++r)
#pragma unroll
        for (int h = 0; h < GT; ++h) {
          const float t = group_sum<LPT>(sc[r][h]);
          sc[r][h] = ok[r] ? t : -INFINITY;
        }

      // online softmax: step max per head (uniform across the wave)
      bool grow = false;
      float mn[GT];
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        float t = sc[0][h];
#pragma unroll
        for (int r = 1; r < ROWS; ++r) t = fmaxf(t, sc[r][h]);
        t = stride_max<LPT>(t);
        mn[h] = fmaxf(m[h], t);
        grow |= mn[h] > m[h];
      }
      if (grow) {
#pragma unroll
        for (int h = 0; h < GT; ++h) {
          const float al = exp2_rel(m[h], mn[h]);
          m[h] = mn[h];
          lsum[h] *= al;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] *= al;
        }
      }

      // weights and the weighted sum of V
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        if (ok[r]) {
          float vv[EPL];
          decode_raw<QT, NDW>(vr[r], vv);
#pragma unroll
          for (int h = 0; h < GT; ++h) {
            const float pr = exp2_rel(sc[r][h], m[h]);
            lsum[h] += pr;
            const float w = pr * vs[r];
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(w, vv[e], acc[h][e]);
          }
        }
      }
    }

    // ---- merge the rows held by other lanes, then the four waves ------------------
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      lsum[h] = stride_sum<LPT>(lsum[h]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = stride_sum<LPT>(acc[h][e]);
    }
    __syncthreads();  // s_red / s_ml of the previous item are free
    if (tsub == 0)
#pragma unroll
      for (int h = 0; h < GT; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) s_red[(wave * GT + h) * D + d0 + e] = acc[h][e];
    if (lane == 0)
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        s_ml[wave][h][0] = m[h];
        s_ml[wave][h][1] = lsum[h];
      }
    __syncthreads();
    if (tid < GT) {
      float M = s_ml[0][tid][0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_ml[w][tid][0]);
      float Ls = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) Ls += exp2_rel(s_ml[w][tid][0], M) * s_ml[w][tid][1];
      s_hm[tid][0] = M;
      s_hm[tid][1] = Ls;
    }
    __syncthreads();
    for (int idx = tid; idx < GT * D; idx += kThreads) {
      const int h = idx / D, d = idx - h * D;
      const float M = s_hm[h][0];
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += exp2_rel(s_ml[w][h][0], M) * s_red[(w * GT + h) * D + d];
      if (nc == 1) {
        const float Ls = s_hm[h][1];
        const int64_t orow = (int64_t)b * a.n_q_heads + h0 + h;
        a.out[orow * D + d] = (uint16_t)bf16_rne(Ls > 0.0f ? v / Ls : 0.0f);
        if (d == 0 && a.lse) a.lse[orow] = (M == -INFINITY) ? -INFINITY : (M + log2f(Ls)) * kLn2;
      } else {
        p.part_acc[((int64_t)item * GT + h) * D + d] = v;
        if (d == 0) {
          p.part_ml[((int64_t)item * GT + h) * 2 + 0] = M;
          p.part_ml[((int64_t)item * GT + h) * 2 + 1] = s_hm[h][1];
        }
      }
    }
    if (nc == 1) continue;

    // ---- the last item of this (sequence, kv head, head group) merges ---------------
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const int old = atomicAdd(&p.count[(int64_t)b * units + u], 1);
      s_last = (old == nc - 1);
    }
    __syncthreads();
    if (!s_last) continue;
    __threadfence();
    const int first = s_prefix[b] + u;  // item of chunk c: first + c * units
    // chunk maxima -> per-head max and sum; weights kept in s_red [nc][GT]
    for (int idx = tid; idx < nc * GT; idx += kThreads) {
      const int c = idx / GT, h = idx - c * GT;
      s_red[idx] = p.part_ml[((int64_t)(first + c * units) * GT + h) * 2];
    }
    __syncthreads();
    for (int h = wave; h < GT; h += kWaves) {
      float M = -INFINITY;
      for (int c = lane; c < nc; c += 64) M = fmaxf(M, s_red[c * GT + h]);
      M = stride_max<1>(M);
      float Ls = 0.0f;
      for (int c = lane; c < nc; c += 64) {
        const float w = exp2_rel(s_red[c * GT + h], M);
        Ls += w * p.part_ml[((int64_t)(first + c * units) * GT + h) * 2 + 1];
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
      float v0 = 0.0f, v1 = 0.0f, v2 = 0.0f, v3 = 0.0f;
      int c = 0;
      for (; c + 4 <= nc; c += 4) {
        v0 += s_red[(c + 0) * GT + h] * p.part_acc[((int64_t)(first + (c + 0) * units) * GT + h) * D + d];
        v1 += s_red[(c + 1) * GT + h] * p.part_acc[((int64_t)(first + (c + 1) * units) * GT + h) * D + d];
        v2 += s_red[(c + 2) * GT + h] * p.part_acc[((int64_t)(first + (c + 2) * units) * GT + h) * D + d];
        v3 += s_red[(c + 3) * GT + h] * p.part_acc[((int64_t)(first + (c + 3) * units) * GT + h) * D + d];
      }
      for (; c < nc; ++c)
        v0 += s_red[c * GT + h] * p.part_acc[((int64_t)(first + c * units) * GT + h) * D + d];
      const float v = (v0 + v1) + (v2 + v3);
      const float M = s_hm[h][0], Ls = s_hm[h][1];
      const int64_t orow = (int64_t)b * a.n_q_heads + h0 + h;
      a.out[orow * D + d] = (uint16_t)bf16_rne(Ls > 0.0f ? v / Ls : 0.0f);
      if (d == 0 && a.lse) a.lse[orow] = (M == -INFINITY) ? -INFINITY : (M + log2f(Ls)) * kLn2;
    }
    if (tid == 0) p.count[(int64_t)b * units + u] = 0;  // ready for the next call
  }
}

template <int QT, int D, int GT>
hipError_t launch_one(const GqaParams& gp, int grid, hipStream_t s) {
  const size_t dyn = (size_t)(gp.a.batch + 1) * sizeof(int);
  gqa_decode_kernel<QT, D, GT><<<grid, kThreads, dyn, s>>>(gp);
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

}  // namespace

hipError_t launch_gqa_decode(const DecodeArgs& a, const DecodePlan& plan, int num_cus,
                             hipStream_t s) {
  char* ws = static_cast<char*>(a.workspace);
  GqaParams gp;
  gp.a = a;
  gp.gt = plan.gt;
  gp.n_hg = plan.n_hg;
  gp.item_tokens = plan.item_pages * kPageSize;
  gp.scale_log2 = a.sm_scale * kLog2e;
  gp.prefix = reinterpret_cast<int*>(ws + plan.off_prefix);
  gp.count = reinterpret_cast<int*>(ws + plan.off_count);
  gp.part_ml = reinterpret_cast<float*>(ws + plan.off_ml);
  gp.part_acc = reinterpret_cast<float*>(ws + plan.off_acc);
  int64_t grid = (int64_t)num_cus * 4;
  if (grid > plan.max_items) grid = plan.max_items;
  if (grid < 1) grid = 1;
  switch (a.qtype) {
    case QT_BF16: return launch_d<QT_BF16>(gp, (int)grid, s);
    case QT_FP8: return launch_d<QT_FP8>(gp, (int)grid, s);
    default: return launch_d<QT_Q8>(gp, (int)grid, s);
  }
}

}  // namespace kvq
