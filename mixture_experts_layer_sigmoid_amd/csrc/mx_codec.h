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

// E4M3 (bias 7, 3 mantissa bits, max 448, no inf) code of y.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t code;
  if (a >= 448.f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {  // below the smallest normal 2^-6: grid step 2^-9
    code = static_cast<uint32_t>(rintf(a * 512.f));
  } else {
    const int ex = floor_log2(a);                 // -6 .. 8
    const float m = ldexpf(a, 3 - ex);            // [8, 16)
    const uint32_t q = static_cast<uint32_t>(rintf(m));   // 8 .. 16
    code = static_cast<uint32_t>((ex + 7) << 3) + (q - 8u);
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

// E2M1 (bias 1, 1 mantissa bit, magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6) code.
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 28) & 0x8u;
  const float a = fabsf(y);
  uint32_t code;
  if (a >= 6.f) {
    code = 7u;
  } else if (a < 1.f) {  // subnormal step 0.5; rounding up to 1 gives code 2
    code = static_cast<uint32_t>(rintf(a * 2.f));
  } else {
    const int ex = floor_log2(a);                 // 0 .. 2
    const float m = ldexpf(a, 1 - ex);            // [2, 4)
    const uint32_t q = static_cast<uint32_t>(rintf(m));   // 2 .. 4
    code = static_cast<uint32_t>((ex + 1) << 1) + (q - 2u);
    if (code > 7u) code = 7u;
  }
  return sign | code;
}

// Encode one block of 32 values. E4M3: codes8[0..31] one byte each packed in
// 8 dwords. E2M1: 16 bytes packed in 4 dwords (even element low nibble).
template <bool FP4>
__device__ __forceinline__ uint32_t mx_encode_block(const float* v, uint32_t* out_words) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  uint32_t sbyte;
  const int e = mx_scale_exponent<FP4 ? 2 : 8>(amax, &sbyte);
  if (FP4) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) word |= e2m1_code(ldexpf(v[w * 8 + i], -e)) << (4 * i);
      out_words[w] = word;
    }
  } else {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) word |= e4m3_code(ldexpf(v[w * 4 + i], -e)) << (8 * i);
      out_words[w] = word;
    }
  }
  return sbyte;
}

}  // namespace moe
