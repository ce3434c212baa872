// NVFP4 quantization: per-tensor scales and the block quantizer.
//
// Page "Mistral Large 3 NVFP4 TRTLLM MoE support" (title, Modifications:
// W4A4 NVFP4 MoE). Layout: E2M1 codes two per byte (even element in the low
// nibble), one E4M3 scale per 16 consecutive values along K ([rows, K/16]),
// one fp32 scale g per tensor; value = e2m1 * e4m3 * g. A weight matrix's
// g = amax / (6 * 448) (1 for an all-zero matrix); the block rule is in
// nvfp4_codec.h.
//
// The GEMMs of the NVFP4 layer take the activation operand as its values
// code * scale (exact in bf16, the tensor scale left out and applied to the
// fp32 accumulators), so the quantizer can write those values as well.
#include "common.h"
#include "nvfp4_codec.h"

#include <algorithm>

namespace moe {
namespace {

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += 256 * gridDim.x) p[i] = 0u;
}

// amax of each tensor's chunk, folded into the tensor's slot with an integer
// max of the fp32 bits (non-negative values order like their bits), so the
// result does not depend on the order of the workgroups
template <int F>
__global__ __launch_bounds__(256) void amax_kernel(const void* __restrict__ in, int64_t per_tensor,
                                                   int chunks, uint32_t* __restrict__ out_bits) {
  __shared__ float red[256];
  const int tensor = blockIdx.x / chunks, chunk = blockIdx.x % chunks;
  const int64_t lo = per_tensor * chunk / chunks, hi = per_tensor * (chunk + 1) / chunks;
  const int64_t base = static_cast<int64_t>(tensor) * per_tensor;
  float m = 0.f;
  for (int64_t i = lo + threadIdx.x; i < hi; i += 256) {
    const float v = F == MOE_BF16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(in)[base + i])
                                  : static_cast<const float*>(in)[base + i];
    m = fmaxf(m, fabsf(v));
  }
  red[threadIdx.x] = m;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0) atomicMax(out_bits + tensor, __float_as_uint(red[0]));
}

__global__ __launch_bounds__(256) void amax_to_scale_kernel(float* g, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += 256 * gridDim.x) {
    const float amax = __uint_as_float(reinterpret_cast<uint32_t*>(g)[i]);
    g[i] = amax > 0.f ? amax / 2688.f : 1.f;
  }
}

// one thread per block of 16 values
template <int F>
__global__ __launch_bounds__(256) void quantize_nvfp4_kernel(const void* __restrict__ in, int64_t rows,
                                                             int K, int64_t rows_per_tensor,
                                                             const float* __restrict__ g,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales,
                                                             uint16_t* __restrict__ vals) {
  const int nb = K / 16;
  const int64_t total = rows * nb;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < total; i += 256ll * gridDim.x) {
    const int64_t r = i / nb;
    const int b = static_cast<int>(i % nb);
    float v[16];
    const int64_t off = r * K + 16 * b;
    if constexpr (F == MOE_BF16) {
      const u32x4_t* p = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(in) + off);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4_t q = p[h];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          v[8 * h + 2 * c] = __uint_as_float(q[c] << 16);
          v[8 * h + 2 * c + 1] = __uint_as_float(q[c] & 0xFFFF0000u);
        }
      }
    } else {
      const float* p = static_cast<const float*>(in) + off;
      load8_f32(p, v);
      load8_f32(p + 8, v + 8);
    }
    const float gt = g[r / rows_per_tensor];
    const float d6 = 6.f * gt;
    uint32_t cw[2], vw[8];
    const uint32_t sc = nvfp4_encode_block(v, gt, d6, cw, vals ? vw : nullptr);
    if (codes) *reinterpret_cast<uint2*>(codes + off / 2) = make_uint2(cw[0], cw[1]);
    if (scales) scales[r * nb + b] = static_cast<uint8_t>(sc);
    if (vals) {
      u32x4_t* o = reinterpret_cast<u32x4_t*>(vals + off);
      o[0] = u32x4_t{vw[0], vw[1], vw[2], vw[3]};
      o[1] = u32x4_t{vw[4], vw[5], vw[6], vw[7]};
    }
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_nvfp4_tensor_scale(const void* in, int in_fmt, int n_tensors,
                                      int64_t elems_per_tensor, float* g, hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(n_tensors >= 1 && elems_per_tensor >= 1, MOE_ERR_INVALID_ARG,
              "moe_nvfp4_tensor_scale: need n_tensors >= 1 and elems_per_tensor >= 1");
  MOE_REQUIRE(in_fmt == MOE_BF16 || in_fmt == MOE_F32, MOE_ERR_UNSUPPORTED,
              "moe_nvfp4_tensor_scale: in_fmt must be MOE_BF16 or MOE_F32");
  MOE_REQUIRE(in && g, MOE_ERR_INVALID_ARG, "moe_nvfp4_tensor_scale: null pointer");
  uint32_t* bits = reinterpret_cast<uint32_t*>(g);
  const unsigned zg = static_cast<unsigned>(std::min(1024, (n_tensors + 255) / 256));
  hipLaunchKernelGGL(zero_u32_kernel, dim3(zg), dim3(256), 0, stream, bits, n_tensors);
  const int chunks = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(
      (elems_per_tensor + 65535) / 65536, std::max<int64_t>(1, 4096 / n_tensors))));
  const dim3 grid(static_cast<unsigned>(n_tensors * chunks));
  if (in_fmt == MOE_BF16)
    hipLaunchKernelGGL(amax_kernel<MOE_BF16>, grid, dim3(256), 0, stream, in, elems_per_tensor, chunks,
                       bits);
  else
    hipLaunchKernelGGL(amax_kernel<MOE_F32>, grid, dim3(256), 0, stream, in, elems_per_tensor, chunks,
                       bits);
  hipLaunchKernelGGL(amax_to_scale_kernel, dim3(zg), dim3(256), 0, stream, g, n_tensors);
  return check_launch("moe_nvfp4_tensor_scale");
}

extern "C" int moe_quantize_nvfp4(const void* in, int in_fmt, int64_t rows, int K,
                                  int64_t rows_per_tensor, const float* g, uint8_t* codes,
                                  uint8_t* scales, void* vals, hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(rows >= 0 && K > 0 && K % 16 == 0 && rows_per_tensor >= 1, MOE_ERR_INVALID_ARG,
              "moe_quantize_nvfp4: need rows >= 0, K a positive multiple of 16, rows_per_tensor >= 1");
  MOE_REQUIRE(in_fmt == MOE_BF16 || in_fmt == MOE_F32, MOE_ERR_UNSUPPORTED,
              "moe_quantize_nvfp4: in_fmt must be MOE_BF16 or MOE_F32");
  if (rows == 0) return MOE_OK;
  MOE_REQUIRE(in && g && (codes || scales || vals), MOE_ERR_INVALID_ARG,
              "moe_quantize_nvfp4: null input or tensor scales, or no output");
  MOE_REQUIRE(aligned16(in) && (!vals || aligned16(vals)) &&
                  (!codes || (reinterpret_cast<uintptr_t>(codes) & 7u) == 0),
              MOE_ERR_ALIGNMENT,
              "moe_quantize_nvfp4: in and vals must be 16-byte, codes 8-byte aligned");
  const int64_t total = rows * (K / 16);
  const unsigned grid = static_cast<unsigned>(std::min<int64_t>(16384, (total + 255) / 256));
  if (in_fmt == MOE_BF16)
    hipLaunchKernelGGL(quantize_nvfp4_kernel<MOE_BF16>, dim3(grid), dim3(256), 0, stream, in, rows, K,
                       rows_per_tensor, g, codes, scales, static_cast<uint16_t*>(vals));
  else
    hipLaunchKernelGGL(quantize_nvfp4_kernel<MOE_F32>, dim3(grid), dim3(256), 0, stream, in, rows, K,
                       rows_per_tensor, g, codes, scales, static_cast<uint16_t*>(vals));
  return check_launch("moe_quantize_nvfp4");
}
