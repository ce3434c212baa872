// Shared helpers of the gfx950 MoE library: status reporting, storage-type
// conversion, MFMA wrappers and launch geometry.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <string>

#include "moe_mi355x.h"

namespace moe {

// ---- status ----------------------------------------------------------------
void set_error(const std::string& msg);
void clear_error();
int fail(int status, const std::string& msg);
int check_launch(const char* what);

#define MOE_REQUIRE(cond, status, msg)                 \
  do {                                                  \
    if (!(cond)) return ::moe::fail((status), (msg));   \
  } while (0)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---- chip geometry -----------------------------------------------------------
// MI355X: 256 compute units in 8 XCDs of 32; workgroups are dispatched to the
// XCDs round-robin by workgroup index.
constexpr int kNumXcd = 8;
constexpr int kNumCu = 256;

// ---- device-side scalar helpers ---------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16_bits(lo)) |
         (static_cast<uint32_t>(f32_to_bf16_bits(hi)) << 16);
}

// Eight consecutive fp32 values as two 16-byte accesses (p 16-byte aligned).
__device__ __forceinline__ void load8_f32(const float* p, float* v) {
  const f32x4_t a = reinterpret_cast<const f32x4_t*>(p)[0];
  const f32x4_t b = reinterpret_cast<const f32x4_t*>(p)[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}
__device__ __forceinline__ void store8_f32(float* p, const float* v) {
  reinterpret_cast<f32x4_t*>(p)[0] = f32x4_t{v[0], v[1], v[2], v[3]};
  reinterpret_cast<f32x4_t*>(p)[1] = f32x4_t{v[4], v[5], v[6], v[7]};
}

// s_waitcnt that waits until at most n vector-memory operations are
// outstanding (gfx9 encoding: vmcnt in bits [3:0] and [15:14]; expcnt and
// lgkmcnt left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  constexpr int imm = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
  __builtin_amdgcn_s_waitcnt(imm);
}

__device__ __forceinline__ void wait_lgkmcnt0() {
  // vmcnt max (63), expcnt max (7), lgkmcnt 0
  constexpr int imm = 0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8);
  __builtin_amdgcn_s_waitcnt(imm);
}

// Map a workgroup index to (xcd, slot within that XCD, slots per XCD), for a
// grid whose size is a multiple of kNumXcd.
struct XcdSlot {
  int xcd, slot, nslots;
};
__device__ __forceinline__ XcdSlot xcd_slot() {
  XcdSlot s;
  s.xcd = blockIdx.x % kNumXcd;
  s.slot = blockIdx.x / kNumXcd;
  s.nslots = gridDim.x / kNumXcd;
  return s;
}

}  // namespace moe
