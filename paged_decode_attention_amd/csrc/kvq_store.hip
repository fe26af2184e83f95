// kvq_store.hip -- quantize-on-store and gather-dequantize kernels (gfx950).
//
// Sources: [PR103] "feat(kvcache): 8-bit KV cache (q8_0 / fp8_e4m3) behind
// --kv-cache-dtype" (§What; review comment §"A bug on sm_89"), [PR113]
// "feat(kvcache): 8-bit DSV4 window/compressed KV behind --kv-cache-dtype"
// (§What this adds).
//
// Mapping: a lane pair owns one 32-element block, 16 elements per lane (two
// 16-byte loads of bf16 per tensor).  The block max-abs is one DPP xor-1 max
// across the pair; both lanes derive the same fp16 scale, quantize their 16
// elements and write 16 code bytes in one store; the even lane writes the
// 2-byte scale.  K and V of the same (token, head, block) are handled by the
// same lane, so a thread keeps four independent 16-byte loads in flight.
// Workgroups are remapped so that each XCD takes one contiguous run of
// tokens (xcd_block).
//
// Infinite elements saturate: the block max is then infinite, its scale is
// held at 65504, the infinite element stores +-M and the others their
// quotient by 65504.  NaN elements are not supported.
//
// The cast types (a per-tensor scale of 1.0, [PR126] "Add fp8 KV-cache
// quantization (--kv-dtype)" §How it works) take the same lanes without the
// block max or a scale: each element is clamped to the format's largest
// finite magnitude (448 e4m3, 57344 e5m2) and rounded to nearest even by the
// packed e4m3 / e5m2 conversion.
//
// Rounding: the code is the round-to-nearest-even e4m3 value (hardware packed
// conversion) or the half-away-from-zero integer (q8_0) of the clamped
// quotient x / s, where the quotient is the correctly rounded fp32 one.  This
// is the store the review comment on [PR103] asks for; a truncating
// intermediate fp16 step (the bug it describes) is never taken.
//
// The quotient is formed as q0 = x * rcp(s) followed by one residual
// correction, q = q0 + fma(-s, q0, x) * rcp(s), instead of the full IEEE
// division sequence.  That gives the same codes: x has an 8-bit and s an
// 11-bit significand, so x / s is either exactly a rounding midpoint of the
// code grid (a value with at most 5 significant bits, which the corrected
// quotient reproduces exactly) or lies at least 2^-18 (relative) away from
// every midpoint, far more than the corrected quotient's error of one fp32
// ulp; the clamp to +-M is monotone, and the sign is taken from x (so -0
// stays -0).  Every (block max, element) pair of bf16 values is checked
// against the oracle's division on the GPU.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;

struct StoreGrid {
  FastDiv per_token;  // lanes per token = n_heads * lanes per head row
  FastDiv per_head;   // lanes per head row = nb * 2 (8-bit) or head_dim / 8 (bf16)
  uint32_t n_lanes;
};

// Workgroups are dealt to the 8 XCDs in turn (block b runs on XCD b % 8).
// Give each XCD one contiguous run of logical blocks instead, so that the
// consecutive tokens of a page -- whose 128-byte scale rows and code rows
// share cache lines -- are written through one L2 and leave it as whole
// lines.  A bijection on [0, n): XCD x holds n / 8 blocks, plus one if
// x < n % 8.
__device__ __forceinline__ uint32_t xcd_block(uint32_t b, uint32_t n) {
  const uint32_t q = n >> 3, r = n & 7u, x = b & 7u;
  return x * q + (x < r ? x : r) + (b >> 3);
}

// The slot of a token: from the slot map, or in append mode from the
// sequence's length and page table (-1: nothing to store).
__device__ __forceinline__ int32_t token_slot(const StoreArgs& a, int64_t token) {
  if (!a.seq_lens) return a.slots[token];
  const int32_t L = a.seq_lens[token];
  if (L < 1 || (int64_t)L > (int64_t)a.max_pages * a.page_size) return -1;
  const int32_t P = a.page_table[token * a.pt_stride + (L - 1) / a.page_size];
  if (P < 0 || (int64_t)P >= a.num_pages) return -1;
  return P * a.page_size + (L - 1) % a.page_size;
}

template <int QT>
__global__ __launch_bounds__(kThreads) void store_kernel(StoreArgs a, StoreGrid g) {
  // 8-bit formats: 16 elements per lane, a 32-element block on a lane pair;
  // bf16: 8 elements (one 16-byte piece) per lane
  constexpr int E = (QT == QT_BF16) ? 8 : 16;
  const uint32_t lane = xcd_block(blockIdx.x, gridDim.x) * kThreads + threadIdx.x;
  // A lane pair must stay together for the DPP max, so no early return
  // before it; out-of-range lanes only skip their memory accesses.
  const bool in_range = lane < g.n_lanes;
  const uint32_t l = in_range ? lane : 0u;
  const uint32_t token = g.per_token.div(l);
  const uint32_t r0 = l - token * g.per_token.d;
  const uint32_t h = g.per_head.div(r0);
  const uint32_t r1 = r0 - h * g.per_head.d;  // piece of E elements within the row
  const int nb = a.head_dim >> 5;

  const int32_t slot = in_range ? token_slot(a, token) : -1;
  const int64_t cap = a.num_pages * (int64_t)a.page_size;
  const bool valid = slot >= 0 && (int64_t)slot < cap;

  const int64_t col = (int64_t)r1 * E;
  const int64_t src_off = (int64_t)token * a.stride + (int64_t)h * a.head_dim + col;
  const int64_t page = valid ? slot / a.page_size : 0;
  const int64_t off = valid ? slot - page * a.page_size : 0;
  const int64_t row = (page * a.n_heads + h) * a.page_size + off;

  // the source rows exist for every token: all loads are issued at once,
  // without waiting for the slot
  constexpr int NP = E / 8;  // 16-byte source pieces per lane
  uint4 raws[2][NP];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int p = 0; p < NP; ++p)
      raws[t][p] = a.src[t] ? *reinterpret_cast<const uint4*>(a.src[t] + src_off + 8 * p)
                            : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (a.src[t] == nullptr) continue;  // uniform: V absent
    if constexpr (QT == QT_BF16) {
      if (valid) *reinterpret_cast<uint4*>(a.pool[t] + (row * a.head_dim + col) * 2) = raws[t][0];
    } else {
      const uint32_t bf[8] = {raws[t][0].x, raws[t][0].y, raws[t][0].z, raws[t][0].w,
                              raws[t][1].x, raws[t][1].y, raws[t][1].z, raws[t][1].w};
      uint32_t codes[4];
      uint16_t sbits;
      quantize_piece<QT, 16>(bf, codes, &sbits);
      if constexpr (qt_scaled(QT))
        if (valid && (r1 & 1u) == 0) a.scales[t][row * nb + (r1 >> 1)] = sbits;
      if (valid)
        *reinterpret_cast<uint4*>(a.pool[t] + row * a.head_dim + col) =
            make_uint4(codes[0], codes[1], codes[2], codes[3]);
    }
  }
}

// ---- dequant: 8 codes per lane -> 8 bf16 (one 16-byte store) -------------------

struct DequantGrid {
  FastDiv per_token;  // lanes per token = n_heads * head_dim / 8
  FastDiv per_head;   // head_dim / 8
  uint32_t n_lanes;
};

template <int QT>
__global__ __launch_bounds__(kThreads) void dequant_kernel(DequantArgs a, DequantGrid g) {
  const uint32_t lane = blockIdx.x * kThreads + threadIdx.x;
  if (lane >= g.n_lanes) return;
  const uint32_t token = g.per_token.div(lane);
  const uint32_t r0 = lane - token * g.per_token.d;
  const uint32_t h = g.per_head.div(r0);
  const uint32_t e8 = r0 - h * g.per_head.d;  // which group of 8 elements
  const int32_t slot = a.slots[token];
  const int64_t cap = a.num_pages * (int64_t)a.page_size;
  uint4 outv = make_uint4(0, 0, 0, 0);
  if (slot >= 0 && (int64_t)slot < cap) {
    const int64_t page = slot / a.page_size, off = slot - page * a.page_size;
    const int64_t row = (page * a.n_heads + h) * a.page_size + off;
    if constexpr (QT == QT_BF16) {
      outv = *reinterpret_cast<const uint4*>(a.pool + (row * a.head_dim + e8 * 8) * 2);
    } else {
      const uint2 raw = *reinterpret_cast<const uint2*>(a.pool + row * a.head_dim + e8 * 8);
      const float s =
          qt_scaled(QT) ? f16_bits_to_f32(a.scales[row * (a.head_dim >> 5) + (e8 >> 2)]) : 1.0f;
      float x[8];
      decode_dword<QT>(raw.x, x);
      decode_dword<QT>(raw.y, x + 4);
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = bf16_rne(x[2 * i] * s) | (bf16_rne(x[2 * i + 1] * s) << 16);  // products exact
      outv = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  *reinterpret_cast<uint4*>(a.out + ((int64_t)token * a.n_heads + h) * a.head_dim + e8 * 8) = outv;
}

// ---- the 656-byte MLA row ------------------------------------------------------------
// One wave per token: lane l quantizes latent elements 8l .. 8l+7, the 16
// lanes of tile j = l / 16 share its maximum; the tile scale is amax / 448 as
// an IEEE fp32 division and each element's quotient x / s too (a 24-bit scale
// leaves no margin for a reciprocal shortcut); clamp, then the packed RNE
// conversion.  A zero tile stores scale 0 and zero codes.  Lanes 0-15 copy
// the 64 rope elements (8 bytes each).
__global__ __launch_bounds__(kThreads) void store_dsm_kernel(StoreArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t token = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (token >= a.n_tokens) return;  // uniform over the wave
  const int32_t slot = token_slot(a, token);
  if (slot < 0 || (int64_t)slot >= a.num_pages * (int64_t)a.page_size) return;
  const uint16_t* src = a.src[0] + token * a.stride;
  const uint4 raw = *reinterpret_cast<const uint4*>(src + 8 * lane);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float x[8], m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
    m = fmaxf(m, fmaxf(fabsf(x[2 * i]), fabsf(x[2 * i + 1])));
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));  // the tile's 16 lanes
  const float sc = m / 448.0f;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (sc > 0.0f) ? x[i] / sc : 0.0f;
  uint32_t c[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) c[k] = e4m3x4_clamped(v[4 * k + 0], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
  uint8_t* row = a.pool[0] + (int64_t)slot * kDsmRow;  // n_heads = 1
  *reinterpret_cast<uint2*>(row + 8 * lane) = make_uint2(c[0], c[1]);
  if ((lane & 15) == 0) *reinterpret_cast<float*>(row + kDsmLatent + 4 * (lane >> 4)) = sc;
  if (lane < 16)
    *reinterpret_cast<uint2*>(row + kDsmLatent + 16 + 8 * lane) =
        *reinterpret_cast<const uint2*>(src + kDsmLatent + 4 * lane);
}

// bf16 of one code x its fp32 tile scale, rounded once: the fp32 product p is
// exact up to the fma residual r; only when p falls exactly on a bf16
// rounding midpoint does r decide the direction.
__device__ __forceinline__ uint32_t bf16_of_product(float x, float s) {
  const float p = x * s;
  const float r = fmaf(x, s, -p);
  uint32_t b = __float_as_uint(p);
  if ((b & 0xffffu) == 0x8000u && r != 0.0f) {
    // exact value beyond the midpoint (away from zero) rounds up in
    // magnitude, below it down
    const bool away = (r > 0.0f) == (p > 0.0f);
    return away ? (b + 0x8000u) >> 16 : (b - 0x8000u) >> 16;
  }
  return bf16_rne(p);
}

// One wave per token: lane l decodes latent elements 8l .. 8l+7; lanes 0-7
// copy 8 rope elements each.
__global__ __launch_bounds__(kThreads) void dequant_dsm_kernel(DequantArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t token = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (token >= a.n_tokens) return;  // uniform over the wave
  const int32_t slot = a.slots[token];
  uint16_t* out = a.out + token * kMlaDqk;
  uint4 lat = make_uint4(0, 0, 0, 0), rope = make_uint4(0, 0, 0, 0);
  if (slot >= 0 && (int64_t)slot < a.num_pages * (int64_t)a.page_size) {
    const uint8_t* row = a.pool + (int64_t)slot * kDsmRow;
    const uint2 raw = *reinterpret_cast<const uint2*>(row + 8 * lane);
    const float s = *reinterpret_cast<const float*>(row + kDsmLatent + 4 * (lane >> 4));
    float x[8];
    decode_dword<QT_DSM>(raw.x, x);
    decode_dword<QT_DSM>(raw.y, x + 4);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = bf16_of_product(x[2 * i], s) | (bf16_of_product(x[2 * i + 1], s) << 16);
    lat = make_uint4(o[0], o[1], o[2], o[3]);
    if (lane < 8) rope = *reinterpret_cast<const uint4*>(row + kDsmLatent + 16 + 16 * lane);
  }
  *reinterpret_cast<uint4*>(out + 8 * lane) = lat;
  if (lane < 8) *reinterpret_cast<uint4*>(out + kDsmLatent + 8 * lane) = rope;
}

}  // namespace

hipError_t launch_store(const StoreArgs& a, hipStream_t s) {
  if (a.n_tokens > 0 && a.qtype == QT_DSM) {
    const int64_t blocks = (a.n_tokens + kThreads / 64 - 1) / (kThreads / 64);
    store_dsm_kernel<<<(unsigned)blocks, kThreads, 0, s>>>(a);
    return hipGetLastError();
  }
  if (a.n_tokens == 0) return hipSuccess;
  const int nb = a.head_dim / 32;
  // 8-bit formats: a 32-element block = 2 lanes of 16 elements; bf16 pools
  // are copied in 16-byte pieces of 8 elements.
  const uint32_t per_head = (uint32_t)(a.qtype == QT_BF16 ? a.head_dim / 8 : nb * 2);
  const uint32_t per_token = per_head * (uint32_t)a.n_heads;
  // keep every launch below 2^31 lanes
  const int64_t max_tokens = ((int64_t)1 << 31) / per_token;
  for (int64_t t0 = 0; t0 < a.n_tokens; t0 += max_tokens) {
    StoreArgs sub = a;
    const int64_t n = (a.n_tokens - t0 < max_tokens) ? a.n_tokens - t0 : max_tokens;
    sub.n_tokens = n;
    if (a.seq_lens) {
      sub.seq_lens = a.seq_lens + t0;
      sub.page_table = a.page_table + t0 * a.pt_stride;
    } else {
      sub.slots = a.slots + t0;
    }
    for (int t = 0; t < 2; ++t)
      if (sub.src[t]) sub.src[t] = a.src[t] + t0 * a.stride;
    StoreGrid g;
    g.per_token = FastDiv(per_token);
    g.per_head = FastDiv(per_head);
    g.n_lanes = (uint32_t)(n * per_token);
    const uint32_t blocks = (g.n_lanes + kThreads - 1) / kThreads;
    switch (a.qtype) {
      case QT_BF16: store_kernel<QT_BF16><<<blocks, kThreads, 0, s>>>(sub, g); break;
      case QT_FP8: store_kernel<QT_FP8><<<blocks, kThreads, 0, s>>>(sub, g); break;
      case QT_FP8C: store_kernel<QT_FP8C><<<blocks, kThreads, 0, s>>>(sub, g); break;
      case QT_BF8C: store_kernel<QT_BF8C><<<blocks, kThreads, 0, s>>>(sub, g); break;
      default: store_kernel<QT_Q8><<<blocks, kThreads, 0, s>>>(sub, g); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Test export: the e4m3 encoder over a range of fp32 bit patterns, four
// consecutive patterns per thread (count is a multiple of 4).
__global__ __launch_bounds__(kThreads) void debug_e4m3_kernel(uint32_t first, uint32_t quads,
                                                              uint32_t* out) {
  const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= quads) return;
  const uint32_t b = first + 4 * i;
  out[i] = e4m3x4_clamped(__uint_as_float(b), __uint_as_float(b + 1), __uint_as_float(b + 2),
                          __uint_as_float(b + 3));  // the clamp is the identity on [-448, 448]
}

hipError_t launch_debug_e4m3(uint32_t first, int64_t count, uint8_t* out, hipStream_t s) {
  for (int64_t done = 0; done < count;) {
    const int64_t n = (count - done < ((int64_t)1 << 30)) ? count - done : ((int64_t)1 << 30);
    const uint32_t quads = (uint32_t)(n / 4);
    debug_e4m3_kernel<<<(quads + kThreads - 1) / kThreads, kThreads, 0, s>>>(
        first + (uint32_t)done, quads, reinterpret_cast<uint32_t*>(out + done));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    done += n;
  }
  return hipSuccess;
}

hipError_t launch_dequant(const DequantArgs& a, hipStream_t s) {
  if (a.n_tokens == 0) return hipSuccess;
  if (a.qtype == QT_DSM) {
    const int64_t blocks = (a.n_tokens + kThreads / 64 - 1) / (kThreads / 64);
    dequant_dsm_kernel<<<(unsigned)blocks, kThreads, 0, s>>>(a);
    return hipGetLastError();
  }
  const uint32_t per_head = (uint32_t)(a.head_dim / 8);
  const uint32_t per_token = per_head * (uint32_t)a.n_heads;
  const int64_t max_tokens = ((int64_t)1 << 31) / per_token;
  for (int64_t t0 = 0; t0 < a.n_tokens; t0 += max_tokens) {
    DequantArgs sub = a;
    const int64_t n = (a.n_tokens - t0 < max_tokens) ? a.n_tokens - t0 : max_tokens;
    sub.n_tokens = n;
    sub.slots = a.slots + t0;
    sub.out = a.out + t0 * per_token * 8;
    DequantGrid g;
    g.per_token = FastDiv(per_token);
    g.per_head = FastDiv(per_head);
    g.n_lanes = (uint32_t)(n * per_token);
    const uint32_t blocks = (g.n_lanes + kThreads - 1) / kThreads;
    switch (a.qtype) {
      case QT_BF16: dequant_kernel<QT_BF16><<<blocks, kThreads, 0, s>>>(sub, g); break;
      case QT_FP8: dequant_kernel<QT_FP8><<<blocks, kThreads, 0, s>>>(sub, g); break;
      case QT_FP8C: dequant_kernel<QT_FP8C><<<blocks, kThreads, 0, s>>>(sub, g); break;
      case QT_BF8C: dequant_kernel<QT_BF8C><<<blocks, kThreads, 0, s>>>(sub, g); break;
      default: dequant_kernel<QT_Q8><<<blocks, kThreads, 0, s>>>(sub, g); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kvq
