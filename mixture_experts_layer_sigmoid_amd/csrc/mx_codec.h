// MX block encoding on the device: E8M0 block scale + E4M3 / E2M1 element
// codes for one block of 32 fp32 values.
//
// Rule (OCP MX v1.0 conventions; the MoE pages name MXFP8 / 4-bit W4A4
// recipes but print no encoding): scale exponent e = floor(log2 amax) -
// emax_elem (8 for E4M3, 2 for E2M1) clamped to [-127, 127], scale byte
// e + 127 (0 when amax == 0); each element is v * 2^-e rounded to the
// nearest element-grid value with ties to the even code, saturated to the
// largest finite value, keeping v's sign bit. Every step is exact in fp32
// (power-of-two scaling, rintf in round-to-nearest-even mode), so the codes
// are a pure function of the input bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// floor(log2(a)) for finite a > 0, including fp32 subnormals.
__device__ __forceinline__ int floor_log2(float a) {
  uint32_t u = __float_as_uint(a) & 0x7FFFFFFFu;
  int field = static_cast<int>(u >> 23);
  if (field != 0) return field - 127;
  return (31 - __clz(static_cast<int>(u))) - 149;
}

template <int EMAX>
__device__ __forceinline__ int mx_scale_exponent(float amax, uint32_t* scale_byte) {
  if (!(amax > 0.f)) {
    *scale_byte = 0;
    return -127;
  }
  int e = floor_log2(amax) - EMAX;
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  *scale_byte = static_cast<uint32_t>(e + 127);
  return e;
}

// E4M3 (bias 7, 3 mantissa bits, max 448, no inf) code of y, |y| < 2^9.
// Branch-free: at or above the smallest normal 2^-6 the fp32 bits are
// rounded to 3 mantissa bits with ties to even (a carry correctly bumps the
// exponent), and the code is the rounded exponent/mantissa field rebased to
// bias 7; below it the grid step is 2^-9 and the code is rint(|y| * 512),
// which reaches 8 (= 2^-6, the first normal code) when it rounds up. Codes
// above the largest finite value 448 (0x7E) saturate.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
  const int normal = static_cast<int>(r >> 20) - ((127 - 7) << 3);
  const uint32_t sub = static_cast<uint32_t>(rintf(__uint_as_float(a) * 512.f));
  uint32_t code = a < 0x3C800000u ? sub : static_cast<uint32_t>(normal);  // 2^-6
  code = code > 0x7Eu ? 0x7Eu : code;
  return sign | code;
}

// E2M1 (bias 1, 1 mantissa bit, magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6) code
// of y, |y| < 8. Same scheme: at or above 1 the bits are rounded to one
// mantissa bit (ties to even); below 1 the step is 0.5 and the code is
// rint(|y| * 2) (2 = the code of 1.0); above 6 (code 7) saturates.
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 28) & 0x8u;
  const uint32_t a = u & 0x7FFFFFFFu;
  const uint32_t r = a + 0x1FFFFFu + ((a >> 22) & 1u);
  const int normal = static_cast<int>(r >> 22) - ((127 - 1) << 1);
  const uint32_t sub = static_cast<uint32_t>(rintf(__uint_as_float(a) * 2.f));
  uint32_t code = a < 0x3F800000u ? sub : static_cast<uint32_t>(normal);  // 1.0
  code = code > 7u ? 7u : code;
  return sign | code;
}

// Encode one block of 32 values. E4M3: codes8[0..31] one byte each packed in
// 8 dwords. E2M1: 16 bytes packed in 4 dwords (even element low nibble).
// The element codes come from gfx950's pack conversions
// (v_cvt_scalef32_pk_fp4_f32 / _fp8_f32, scale 1.0) applied to v * 2^-e:
// they round to nearest even like e2m1_code / e4m3_code above, and E2M1
// saturates at 6; E4M3 conversion does not saturate (|y| >= 464 would give
// the NaN code), so its input is clamped to +-448 first, which is what the
// rounding rule maps every |y| > 448 to anyway. An in-bounds GPU check
// against e2m1_code / e4m3_code agreed on every code (an fp32 sweep of
// ties, subnormals and saturation, and 200k random blocks).
template <bool FP4>
__device__ __forceinline__ uint32_t mx_encode_block(const float* v, uint32_t* out_words) {
  typedef short v2i16 __attribute__((ext_vector_type(2)));
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  uint32_t sbyte;
  const int e = mx_scale_exponent<FP4 ? 2 : 8>(amax, &sbyte);
  if (FP4) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float* q = v + 8 * w;
      uint32_t word = 0;
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, ldexpf(q[0], -e), ldexpf(q[1], -e), 1.f, 0);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, ldexpf(q[2], -e), ldexpf(q[3], -e), 1.f, 1);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, ldexpf(q[4], -e), ldexpf(q[5], -e), 1.f, 2);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, ldexpf(q[6], -e), ldexpf(q[7], -e), 1.f, 3);
      out_words[w] = word;
    }
  } else {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      float y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        y[i] = __builtin_amdgcn_fmed3f(ldexpf(v[4 * w + i], -e), -448.f, 448.f);
      v2i16 o = {0, 0};
      o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, y[0], y[1], 1.f, false);
      o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, y[2], y[3], 1.f, true);
      out_words[w] = static_cast<uint32_t>(static_cast<uint16_t>(o[0])) |
                     (static_cast<uint32_t>(static_cast<uint16_t>(o[1])) << 16);
    }
  }
  return sbyte;
}

}  // namespace moe
