// NVFP4 block encoding on the device: one block of 16 fp32 values -> E2M1
// codes, an E4M3 block scale, and the operand values code * scale.
//
// Page "Mistral Large 3 NVFP4 TRTLLM MoE support" (title, Modifications: a
// W4A4 NVFP4 MoE) names the format without a recipe; the rule followed is
// the public NVFP4 definition with its two-level scaling: value =
// e2m1(code) * e4m3(s) * g, g one fp32 scale per tensor; for a block,
// s = E4M3 RNE of amax / fp32(6 g) (saturating at 448), codes = E2M1 RNE of
// v / fp32(s g) (saturating at 6, keeping v's sign bit; zero codes when s
// rounds to 0). The divisions are IEEE fp32 divisions and the roundings are
// those of e4m3_code / e2m1_code, so the codes are a pure function of the
// input bits and g.
#pragma once

#include "mx_codec.h"

namespace moe {

// |value| of an E2M1 magnitude code (0, .5, 1, 1.5, 2, 3, 4, 6)
__device__ __forceinline__ float e2m1_magnitude(uint32_t m) {
  return m < 2 ? 0.5f * static_cast<float>(m)
               : (1.f + 0.5f * static_cast<float>(m & 1u)) * __uint_as_float((126u + (m >> 1)) << 23);
}

// E4M3 code (positive) -> fp32 value, exact
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(c), 0);
}

// Encode 16 values with tensor scale g (d6 = fp32(6 * g)). Writes the 16
// codes packed in two dwords (even element in the low nibble), returns the
// E4M3 scale code; vals (optional) receives code * scale as bf16 bits in 8
// dwords (two per dword, even element low), exact.
__device__ __forceinline__ uint32_t nvfp4_encode_block(const float* v, float g, float d6,
                                                       uint32_t* codes, uint32_t* vals) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const float t = amax / d6;
  const uint32_t sc = e4m3_code(fminf(t, 448.f));
  const float s = e4m3_value(sc);
  const float d = s * g;
  uint32_t c[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float q = s > 0.f ? v[i] / d : copysignf(0.f, v[i]);
    c[i] = e2m1_code(__builtin_amdgcn_fmed3f(q, -6.f, 6.f)) | ((__float_as_uint(v[i]) >> 28) & 0x8u);
  }
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= c[8 * w + i] << (4 * i);
    codes[w] = word;
  }
  if (vals) {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      uint32_t pair = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t ci = c[2 * w + h];
        const float val = copysignf(e2m1_magnitude(ci & 7u) * s, (ci & 8u) ? -1.f : 1.f);
        pair |= (__float_as_uint(val) >> 16) << (16 * h);   // exact in bf16
      }
      vals[w] = pair;
    }
  }
  return sc;
}

}  // namespace moe
