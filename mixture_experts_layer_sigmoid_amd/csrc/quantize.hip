// moe_quantize_mx: MX block quantization of [rows, K] along K.
//
// Page "[PyTorch] DeepSeekV3Layer: full MoE transformer layer (MLA +
// DeepSeek MoE)", Performance section, "Where the time goes" table: MXFP8
// quantization of the received rows (group quantize) and of dense GEMM
// inputs (cast only). The encoding rule is in mx_codec.h.
//
// One thread encodes one 32-element block: it reads the block's 64 (bf16) or
// 128 (fp32) contiguous bytes, writes 32 (E4M3) or 16 (E2M1) code bytes and
// one scale byte; consecutive threads take consecutive blocks of a row, so
// every wave reads and writes contiguous memory.
#include "common.h"
#include "mx_codec.h"

namespace moe {
int quantize_mx_columns(const void* in, int64_t rows, int K, int out_fmt, uint8_t* codes,
                        uint8_t* scales, hipStream_t stream);
namespace {

template <int IN_FMT, bool FP4>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const void* __restrict__ in,
                                                            int64_t nblocks, int K,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  const int bpr = K / 32;
  for (int64_t b = blockIdx.x * 256ll + threadIdx.x; b < nblocks; b += 256ll * gridDim.x) {
    const int64_t row = b / bpr;
    const int blk = static_cast<int>(b % bpr);
    float v[32];
    if (IN_FMT == MOE_BF16) {
      const u32x4_t* p = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(in) +
                                                          row * K + blk * 32);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4_t w = p[q];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[q * 8 + 2 * i] = __uint_as_float(w[i] << 16);
          v[q * 8 + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
      }
    } else {
      const f32x4_t* p = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(in) +
                                                          row * K + blk * 32);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        f32x4_t w = p[q];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[q * 4 + i] = w[i];
      }
    }
    uint32_t words[8];
    uint32_t sb = mx_encode_block<FP4>(v, words);
    if (FP4) {
      u32x4_t* o = reinterpret_cast<u32x4_t*>(codes + row * (K / 2) + blk * 16);
      o[0] = u32x4_t{words[0], words[1], words[2], words[3]};
    } else {
      u32x4_t* o = reinterpret_cast<u32x4_t*>(codes + row * K + blk * 32);
      o[0] = u32x4_t{words[0], words[1], words[2], words[3]};
      o[1] = u32x4_t{words[4], words[5], words[6], words[7]};
    }
    scales[row * bpr + blk] = static_cast<uint8_t>(sb);
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_quantize_mx(const void* in, int in_fmt, int64_t rows, int K, int axis,
                               int out_fmt, uint8_t* codes, uint8_t* scales,
                               hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(rows >= 0 && K > 0 && K % 32 == 0, MOE_ERR_INVALID_ARG,
              "moe_quantize_mx: need rows >= 0 and K a positive multiple of 32");
  MOE_REQUIRE(in_fmt == MOE_F32 || in_fmt == MOE_BF16, MOE_ERR_UNSUPPORTED,
              "moe_quantize_mx: in_fmt must be MOE_F32 or MOE_BF16");
  MOE_REQUIRE(out_fmt == MOE_MXFP8_E4M3 || out_fmt == MOE_MXFP4_E2M1, MOE_ERR_UNSUPPORTED,
              "moe_quantize_mx: out_fmt must be an MX format");
  MOE_REQUIRE(axis == 0 || axis == 1, MOE_ERR_INVALID_ARG, "moe_quantize_mx: axis must be 0 or 1");
  MOE_REQUIRE(axis == 0 || in_fmt == MOE_BF16, MOE_ERR_UNSUPPORTED,
              "moe_quantize_mx: axis 1 takes bf16 input");
  MOE_REQUIRE(axis == 0 || rows % 32 == 0, MOE_ERR_INVALID_ARG,
              "moe_quantize_mx: axis 1 needs rows % 32 == 0");
  if (rows == 0) return MOE_OK;
  MOE_REQUIRE(in && codes && scales, MOE_ERR_INVALID_ARG, "moe_quantize_mx: null pointer");
  MOE_REQUIRE(aligned16(in) && aligned16(codes), MOE_ERR_ALIGNMENT,
              "moe_quantize_mx: in and codes must be 16-byte aligned");
  if (axis == 1) return quantize_mx_columns(in, rows, K, out_fmt, codes, scales, stream);
  const int64_t nblocks = rows * (K / 32);
  const int64_t want = (nblocks + 255) / 256;
  const int grid = static_cast<int>(want < 65536 ? want : 65536);
  const bool fp4 = out_fmt == MOE_MXFP4_E2M1;
  if (in_fmt == MOE_BF16) {
    if (fp4)
      hipLaunchKernelGGL((quantize_rows_kernel<MOE_BF16, true>), dim3(grid), dim3(256), 0, stream,
                         in, nblocks, K, codes, scales);
    else
      hipLaunchKernelGGL((quantize_rows_kernel<MOE_BF16, false>), dim3(grid), dim3(256), 0, stream,
                         in, nblocks, K, codes, scales);
  } else {
    if (fp4)
      hipLaunchKernelGGL((quantize_rows_kernel<MOE_F32, true>), dim3(grid), dim3(256), 0, stream,
                         in, nblocks, K, codes, scales);
    else
      hipLaunchKernelGGL((quantize_rows_kernel<MOE_F32, false>), dim3(grid), dim3(256), 0, stream,
                         in, nblocks, K, codes, scales);
  }
  return check_launch("moe_quantize_mx");
}
