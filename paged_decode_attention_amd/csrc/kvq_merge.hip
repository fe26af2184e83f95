// kvq_merge.hip -- split-K merge for the separate-K/V decode kernels when a
// sequence is split into many work items (long contexts, small batches).
//
// Source: [PR113] "feat(kvcache): 8-bit DSV4 window/compressed KV behind
// --kv-cache-dtype" §Testing (split-k decode): partial results over chunks of
// the sequence are combined with their log-sum-exp weights.
//
// Each item of (sequence b, kv head / head group u) left (m_c, l_c) per head
// (log2-domain running max and sum) and acc_c[h][d] (fp32, unnormalized).
// With M = max_c m_c and w_c = 2^(m_c - M):
//   out[h][d] = sum_c w_c acc_c[h][d] / sum_c w_c l_c,  lse = (M + log2 sum_c w_c l_c) ln 2.
// Block = (b, u, head, 32 columns); 32 groups of 8 threads take every 32nd
// chunk, a thread 4 columns (16 columns per block left half the groups idle
// at 32 chunks: 7% slower at head_dim 256); the first chunk rows and every chunk's (m, l)
// are loaded at once, before the weights are formed; the groups' sums meet
// by lane moves inside each wave and one LDS exchange across the waves.  The decode kernels
// merge in their last workgroup instead when the partials of a sequence are
// few (see plan_decode).
#include "kvq_attn.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kCols = 32;                // columns per block
constexpr int kLanesPerRow = kCols / 4;  // a thread takes 4 columns
constexpr int kThreads = 256;
constexpr int kGroups = kThreads / kLanesPerRow;  // chunk rows in flight per block
constexpr int kAhead = 4;                // chunk rows per thread loaded before the weights

struct MergeParams {
  DecodeArgs a;
  int gt, n_hg, units, D;
  const int* prefix;
  const float* part_ml;
  const float* part_acc;
};

__global__ __launch_bounds__(kThreads) void gqa_merge_kernel(MergeParams p) {
  const DecodeArgs& a = p.a;
  const int nd = p.D / kCols;
  int x = blockIdx.x;
  const int dchunk = x % nd;
  x /= nd;
  const int h = x % p.gt;
  x /= p.gt;
  const int u = x % p.units, b = x / p.units;
  const int nc = (p.prefix[b + 1] - p.prefix[b]) / p.units;
  if (nc <= 1) return;  // written by the decode kernel itself
  const int first = p.prefix[b] + u;  // item of chunk c: first + c * units
  __shared__ float s_w[kMergeMaxWeights];
  __shared__ __attribute__((aligned(16))) f32x4 s_red[kGroups][kLanesPerRow];
  __shared__ float s_L;
  __shared__ float s_part[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int G = a.n_q_heads / a.n_kv_heads;
  // (extend attention numbers its units tile-major)
  const int kvh = a.q_start ? u % a.n_kv_heads : u / p.n_hg;
  const int hg = a.q_start ? u / a.n_kv_heads : u - kvh * p.n_hg;
  const int64_t orow = query_row(a, b, kvh, hg * p.gt + h, G);
  if (orow < 0) return;  // a padding column of extend attention
  const int grp = tid / kLanesPerRow, j = tid % kLanesPerRow;
  const float* src = p.part_acc + ((int64_t)first * p.gt + h) * p.D + dchunk * kCols + 4 * j;
  const int64_t cstride = (int64_t)p.units * p.gt * p.D;
  // the first rows' partial sums are in flight while wave 0 forms the weights
  f32x4 xs[kAhead];
#pragma unroll
  for (int k = 0; k < kAhead; ++k) {
    const int c = grp + k * kGroups;
    xs[k] = c < nc ? *reinterpret_cast<const f32x4*>(src + (int64_t)c * cstride)
                   : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // every thread loads the (m, l) of its chunks once (in flight with the rows
  // above); block reductions give M and the weighted sum of l
  constexpr int kMl = (kMergeMaxWeights + kThreads - 1) / kThreads;
  float mc[kMl], lc[kMl];
#pragma unroll
  for (int k = 0; k < kMl; ++k) {
    const int c = tid + k * kThreads;
    mc[k] = -INFINITY;
    lc[k] = 0.0f;
    if (c < nc) {
      const float2 ml = *reinterpret_cast<const float2*>(
          p.part_ml + ((int64_t)(first + c * p.units) * p.gt + h) * 2);
      mc[k] = ml.x;
      lc[k] = ml.y;
    }
  }
  float M = mc[0];
#pragma unroll
  for (int k = 1; k < kMl; ++k) M = fmaxf(M, mc[k]);
  M = stride_max<1>(M);
  if (lane == 0) s_part[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_part[0], s_part[1]), fmaxf(s_part[2], s_part[3]));
  float Ls = 0.0f;
#pragma unroll
  for (int k = 0; k < kMl; ++k) {
    const int c = tid + k * kThreads;
    if (c < nc) {
      const float w = exp2_rel(mc[k], M);
      s_w[c] = w;
      Ls += w * lc[k];
    }
  }
  Ls = stride_sum<1>(Ls);
  __syncthreads();  // every wave has read s_part
  if (lane == 0) s_part[tid >> 6] = Ls;
  __syncthreads();
  if (tid == 0) {
    Ls = s_part[0] + s_part[1] + s_part[2] + s_part[3];
    s_L = Ls;
    if (a.lse && dchunk == 0) a.lse[orow] = (M == -INFINITY) ? -INFINITY : (M + log2f(Ls)) * kLn2;
  }
  __syncthreads();
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kAhead; ++k) {
    const int c = grp + k * kGroups;
    if (c < nc) v += s_w[c] * xs[k];
  }
  for (int c = grp + kAhead * kGroups; c < nc; c += kGroups)
    v += s_w[c] * *reinterpret_cast<const f32x4*>(src + (int64_t)c * cstride);
  // the groups' sums: the 8 groups of a wave (lanes j, j + 8, ..., j + 56)
  // by a DPP row rotation and the two permlane swaps, then the 4 waves
  // through LDS (one barrier)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float x = v[q];
    x += dpp<kRowRor<8>>(x);
    x = sum_xor32(sum_xor16(x));
    v[q] = x;
  }
  if (lane < kLanesPerRow) s_red[tid >> 6][lane] = v;
  __syncthreads();
  if (tid < kLanesPerRow) {
    const f32x4 t = s_red[0][tid] + s_red[1][tid] + s_red[2][tid] + s_red[3][tid];
    const float Ls = s_L;
    const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
    uint16_t* o = a.out + orow * p.D + dchunk * kCols + 4 * tid;
    *reinterpret_cast<u32x2*>(o) = u32x2{pack_bf16x2(t[0] * inv, t[1] * inv), pack_bf16x2(t[2] * inv, t[3] * inv)};
  }
}

}  // namespace

hipError_t launch_gqa_merge(const DecodeArgs& a, const DecodePlan& plan, hipStream_t s) {
  const char* ws = static_cast<const char*>(a.workspace);
  MergeParams mp;
  mp.a = a;
  mp.gt = plan.gt;
  mp.n_hg = plan.n_hg;
  mp.units = a.n_kv_heads * plan.n_hg;
  mp.D = a.head_dim_qk;
  mp.prefix = reinterpret_cast<const int*>(ws + plan.off_prefix);
  mp.part_ml = reinterpret_cast<const float*>(ws + plan.off_ml);
  mp.part_acc = reinterpret_cast<const float*>(ws + plan.off_acc);
  const int64_t grid = (int64_t)a.batch * mp.units * plan.gt * (mp.D / kCols);
  gqa_merge_kernel<<<(int)grid, kThreads, 0, s>>>(mp);
  return hipGetLastError();
}

}  // namespace kvq
