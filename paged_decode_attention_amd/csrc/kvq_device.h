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
