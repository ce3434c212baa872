// Device helpers shared by the grouped GEMM kernels: direct global->LDS
// loads (global and buffer forms), vmcnt waits, the LDS-only workgroup barrier, the swizzled LDS row
// layout and the SwiGLU activation.
#pragma once

#include "common.h"

namespace moe {

__device__ __forceinline__ void lds_load16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)g,
                                   (void __attribute__((address_space(3)))*)lds, 16, 0, 0);
}
__device__ __forceinline__ void lds_load4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)g,
                                   (void __attribute__((address_space(3)))*)lds, 4, 0, 0);
}

// Direct-to-LDS loads through a buffer resource (MUBUF form): lane l's 16
// (or 4) bytes from base + voffset + soffset land at lds + 16 l (4 l). The
// buffer form matters for the LDS operand reads that follow: while a
// global (FLAT) direct-to-LDS load is outstanding the compiler cannot count
// LDS reads in order and waits for all of them (lgkmcnt(0)) before every
// use; with the buffer form its waits stay exact. Offsets past `bytes`
// read as zero instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ void lds_load16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voffset,
                                               uint32_t soffset, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3)))*)lds, 16,
                                           voffset, soffset, 0, 0);
}
__device__ __forceinline__ void lds_load4_buf(__amdgpu_buffer_rsrc_t r, uint32_t voffset,
                                              uint32_t soffset, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3)))*)lds, 4,
                                           voffset, soffset, 0, 0);
}

// Wait until at most n vector-memory operations of this wave are in flight.
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
#define MOE_W(N) case N: wait_vmcnt<N>(); break;
    MOE_W(0) MOE_W(1) MOE_W(2) MOE_W(3) MOE_W(4) MOE_W(5) MOE_W(6) MOE_W(7)
    MOE_W(8) MOE_W(9) MOE_W(10) MOE_W(11) MOE_W(12) MOE_W(13) MOE_W(14) MOE_W(15)
    MOE_W(16) MOE_W(17) MOE_W(18) MOE_W(19) MOE_W(20) MOE_W(21) MOE_W(22) MOE_W(23)
    MOE_W(24) MOE_W(25) MOE_W(26) MOE_W(27) MOE_W(28) MOE_W(29) MOE_W(30) MOE_W(31)
    MOE_W(32) MOE_W(33) MOE_W(34) MOE_W(35) MOE_W(36) MOE_W(37) MOE_W(38) MOE_W(39)
    MOE_W(40) MOE_W(41) MOE_W(42) MOE_W(43) MOE_W(44) MOE_W(45) MOE_W(46) MOE_W(47)
    MOE_W(48) MOE_W(49) MOE_W(50) MOE_W(51) MOE_W(52) MOE_W(53) MOE_W(54) MOE_W(55)
    MOE_W(56) MOE_W(57) MOE_W(58) MOE_W(59) MOE_W(60) MOE_W(61) MOE_W(62)
#undef MOE_W
    default: wait_vmcnt<0>(); break;
  }
}

// Workgroup barrier for the stage pipeline: waits only for this wave's LDS
// operations (not for the global->LDS loads still in flight, which the
// explicit vmcnt accounting covers) before s_barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// byte offset of 16-byte chunk c of row r inside a [rows][128 B] stage tile
// A stage tile stores row r's RB/16 chunks of 16 bytes XOR-permuted by a key
// of r: (r/2)%8 for 128-byte rows, (r/4)%4 for 64-byte rows. Either way any
// 16 consecutive rows put one logical chunk into 16 distinct 16-byte bank
// groups of a 256-byte LDS line, so the MFMA operand reads (16 lanes = 16
// consecutive rows per LDS cycle) are free of bank conflicts.
template <int RB>
__device__ __forceinline__ int swz_key(int r) {
  return RB == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}
template <int RB>
__device__ __forceinline__ int swz(int r, int c) { return r * RB + ((c ^ swz_key<RB>(r)) << 4); }

// silu(g) * u with the hardware exp2 and reciprocal (a few ulp of fp32; the
// result is rounded to bf16 or MX right after)
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * g);
  return g * __builtin_amdgcn_rcpf(1.f + e) * u;
}

}  // namespace moe
