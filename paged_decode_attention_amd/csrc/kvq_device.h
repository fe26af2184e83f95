// kvq_device.h -- small device helpers for the gfx950 kernels of libkvq.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- bf16 / fp16 bit conversions ----------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// ---- 8-bit code decoding --------------------------------------------------------
// e4m3fn: the gfx950 packed conversion decodes two codes (bytes 0,1 or 2,3 of
// a dword) to fp32 exactly.
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* o) {
  f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  o[0] = a.x;
  o[1] = a.y;
  o[2] = b.x;
  o[3] = b.y;
}

// e5m2: the same through the bf8 conversion.
__device__ __forceinline__ void bf8x4_to_f32(uint32_t w, float* o) {
  f32x2 a = __builtin_amdgcn_cvt_pk_f32_bf8(w, false);
  f32x2 b = __builtin_amdgcn_cvt_pk_f32_bf8(w, true);
  o[0] = a.x;
  o[1] = a.y;
  o[2] = b.x;
  o[3] = b.y;
}

// int8: sign-extend each byte.
__device__ __forceinline__ void q8x4_to_f32(uint32_t w, float* o) {
  o[0] = (float)(int32_t)(int8_t)(w & 0xff);
  o[1] = (float)(int32_t)(int8_t)((w >> 8) & 0xff);
  o[2] = (float)(int32_t)(int8_t)((w >> 16) & 0xff);
  o[3] = (float)(int32_t)(int8_t)(w >> 24);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Four 8-bit codes (or two bf16) -> bf16 pairs, exactly: e4m3, e5m2 and int8
// values all fit bf16's 8-bit significand and exponent range.  e4m3 / e5m2
// use the gfx950 scaled packed conversions with scale 1.0; int8 goes through
// fp32.
template <int QT>
__device__ __forceinline__ void decode_dword_bf16x2(uint32_t w, uint32_t* o) {
  if constexpr (QT == QT_FP8 || QT == QT_FP8C || QT == QT_DSM) {
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  } else if constexpr (QT == QT_BF8C) {
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, false));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, true));
  } else if constexpr (QT == QT_Q8) {
    float f[4];
    q8x4_to_f32(w, f);
    // |int8| <= 127 is exact in bf16: truncating the low 16 bits is exact
    o[0] = (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xffff0000u);
    o[1] = (__float_as_uint(f[2]) >> 16) | (__float_as_uint(f[3]) & 0xffff0000u);
  } else {
    o[0] = w;
  }
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// ---- 8-bit float encoding ------------------------------------------------------
// Four fp32 values in [-448, 448] -> four e4m3fn codes in one dword (byte i
// from v_i), rounded to nearest even by the gfx950 packed conversion.  Every
// e4m3 code the library stores comes from here (the block-scaled quotients,
// the cast type and the 656-byte row, each clamped by its caller), and the
// test export kvq_debug_e4m3_encode_range runs it over every fp32 in
// [-448, 448].
__device__ __forceinline__ uint32_t e4m3x4_rne(float v0, float v1, float v2, float v3) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, lo, true);
}
// The same after clamping each value to +-448.
__device__ __forceinline__ uint32_t e4m3x4_clamped(float v0, float v1, float v2, float v3) {
  constexpr float M = 448.0f;
  return e4m3x4_rne(fminf(fmaxf(v0, -M), M), fminf(fmaxf(v1, -M), M), fminf(fmaxf(v2, -M), M),
                    fminf(fmaxf(v3, -M), M));
}

// Two fp32 -> one bf16 pair (round to nearest even), .x in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int QT>
__device__ __forceinline__ void decode_dword(uint32_t w, float* o) {
  if constexpr (QT == QT_FP8 || QT == QT_FP8C || QT == QT_DSM) {
    fp8x4_to_f32(w, o);
  } else if constexpr (QT == QT_BF8C) {
    bf8x4_to_f32(w, o);
  } else if constexpr (QT == QT_Q8) {
    q8x4_to_f32(w, o);
  } else {
    o[0] = bf16_lo(w);
    o[1] = bf16_hi(w);
  }
}

// ---- cross-lane ----------------------------------------------------------------

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// quad_perm DPP swaps within groups of 4 lanes: xor 1 -> [1,0,3,2], xor 2 -> [2,3,0,1].
__device__ __forceinline__ float dpp_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// ---- quantize-on-store of one lane's piece of a row ---------------------------------
// The store kernel and the decode with append both store through these, so an
// appended row holds the same bytes as a stored one.

// Eight elements of a block with the fp16 scale s (as fp32) -> eight 8-bit
// codes in two dwords.  The quotient x / s is x * rcp(s) plus one residual
// correction: x has an 8-bit and s an 11-bit significand, so the exact
// quotient is either a rounding midpoint of the code grid (at most 5
// significant bits, reproduced exactly) or at least 2^-18 (relative) away from
// every midpoint, beyond the corrected quotient's one-ulp error.  The clamp to
// +-M keeps x's sign (-0 stays -0; an infinite element, whose residual is
// inf - inf, stores +-M since fminf(NaN, M) is M).  e4m3: round to nearest
// even by the packed conversion; q8_0: half away from zero.
template <int QT>
__device__ __forceinline__ void quantize8(const float* x, float s, uint32_t* out2) {
  constexpr float M = (QT == QT_Q8) ? 127.0f : 448.0f;
  if (s == 0.0f) {
    out2[0] = 0u;
    out2[1] = 0u;
    return;
  }
  const float r = __builtin_amdgcn_rcpf(s);  // s is a normal fp32 value (an fp16 scale)
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q0 = x[i] * r;
    const float q = fmaf(fmaf(-s, q0, x[i]), r, q0);
    v[i] = copysignf(fminf(fabsf(q), M), x[i]);
  }
  if constexpr (QT == QT_FP8) {
#pragma unroll
    for (int w = 0; w < 2; ++w)
      out2[w] = e4m3x4_rne(v[4 * w + 0], v[4 * w + 1], v[4 * w + 2], v[4 * w + 3]);
  } else {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      uint32_t r = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        int c = (int)roundf(v[4 * w + k]);  // half away from zero, |c| <= 127
        r |= ((uint32_t)c & 0xffu) << (8 * k);
      }
      out2[w] = r;
    }
  }
}

// A lane's E consecutive elements of a row (E/2 bf16 pairs) -> their codes
// (E/4 dwords; a bf16 pool keeps the E/2 dwords as they are) and, for the
// block-scaled types, the fp16 scale bits of the 32-element block.  The block
// spans 32 / E consecutive lanes (a pair for E = 16, four lanes for E = 8),
// all of which must be active: the block max is a DPP max across them.
// Scale: IEEE fp32 amax / M, held at 65504 (an infinite max saturates), then
// fp16 round to nearest even.  Cast types: each element clamped to the
// format's largest finite magnitude (448 e4m3, 57344 e5m2), then the packed
// round-to-nearest-even conversion.
template <int QT, int E>
__device__ __forceinline__ void quantize_piece(const uint32_t* bf, uint32_t* codes,
                                               uint16_t* sbits) {
  static_assert(E == 8 || E == 16, "8 or 16 elements per lane");
  if constexpr (QT == QT_BF16) {
#pragma unroll
    for (int i = 0; i < E / 2; ++i) codes[i] = bf[i];
    *sbits = 0;
  } else {
    float x[E];
#pragma unroll
    for (int i = 0; i < E / 2; ++i) {
      x[2 * i] = bf16_lo(bf[i]);
      x[2 * i + 1] = bf16_hi(bf[i]);
    }
    if constexpr (!qt_scaled(QT)) {
      constexpr float M = (QT == QT_BF8C) ? 57344.0f : 448.0f;
#pragma unroll
      for (int d = 0; d < E / 4; ++d) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = fminf(fmaxf(x[4 * d + i], -M), M);
        if constexpr (QT == QT_BF8C) {
          const int lo = __builtin_amdgcn_cvt_pk_bf8_f32(v[0], v[1], 0, false);
          codes[d] = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(v[2], v[3], lo, true);
        } else {
          codes[d] = e4m3x4_rne(v[0], v[1], v[2], v[3]);
        }
      }
      *sbits = 0;
    } else {
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < E; ++i) amax = fmaxf(amax, fabsf(x[i]));
      amax = fmaxf(amax, dpp_xor1(amax));                        // the block's other lanes
      if constexpr (E == 8) amax = fmaxf(amax, dpp_xor2(amax));
      constexpr float M = (QT == QT_Q8) ? 127.0f : 448.0f;
      float sq = amax / M;           // IEEE fp32 division
      sq = fminf(sq, 65504.0f);      // a quotient past the fp16 range saturates
      const _Float16 sh = (_Float16)sq;  // round to nearest even
      const float s = (float)sh;
#pragma unroll
      for (int i = 0; i < E / 8; ++i) quantize8<QT>(x + 8 * i, s, codes + 2 * i);
      *sbits = __builtin_bit_cast(uint16_t, sh);
    }
  }
}

// ---- division by a runtime constant (unsigned 32-bit, exact) -------------------
// n / d == umulhi(n, m) >> s for all n < 2^31 with m, s from the usual
// round-up reciprocal construction.
struct FastDiv {
  uint32_t d, m, s;
  __host__ __device__ FastDiv() : d(1), m(0), s(0) {}
  __host__ explicit FastDiv(uint32_t div) : d(div) {
    s = 0;
    while ((1ull << s) < div) ++s;
    m = (uint32_t)((((1ull << 32) * ((1ull << s) - div)) / div) + 1);
  }
  __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const {
    return (uint32_t)((((uint64_t)n * m) >> 32) + n) >> s;
  }
};

}  // namespace kvq
