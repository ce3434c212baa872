// moe_combine: routing-weighted reduce of the expert rows back to token
// order, plus the shared expert.
//
// Page "[PyTorch] DeepSeekV3Layer: full MoE transformer layer (MLA +
// DeepSeek MoE)": Performance section, "Where the time goes" table (local
// permute "reduce" back from the expert-major layout) and Description
// (optional shared expert added to the routed output).
//   out[t] = sum_{j<k} w[t, j] * y[row_map[t, j]]  (+ shared[t])
// accumulated in fp32 in slot order j = 0..k-1, then the shared row.
//
// One workgroup per token; each thread owns 8 consecutive columns, reads
// them as one 16-byte (bf16) or two 16-byte (fp32) vectors per row.
#include "common.h"

namespace moe {
namespace {

template <int YF>
__device__ __forceinline__ void load8(const void* base, int64_t off, float* v) {
  if (YF == MOE_BF16) {
    u32x4_t w = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const f32x4_t* p = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(base) + off);
    f32x4_t a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
}

constexpr int kMaxK = 16;  // moe_route's limit on k

template <int YF, int OF>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y,
                                                      const int32_t* __restrict__ row_map,
                                                      const float* __restrict__ w,
                                                      const void* __restrict__ shared, int T, int k,
                                                      int H, void* __restrict__ out) {
  const int t = blockIdx.x;
  const int nvec = H / 8;
  // the token's k rows and weights (uniform across the workgroup): lane j
  // of every wave loads entry j (one memory round trip for all of them),
  // then each is broadcast from its lane
  const int lane = threadIdx.x & 63;
  int rv = 0;
  float wv = 1.f;
  if (lane < k) {
    rv = row_map[static_cast<int64_t>(t) * k + lane];
    if (w) wv = w[static_cast<int64_t>(t) * k + lane];
  }
  int64_t rows[kMaxK];
  float wts[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    rows[j] = j < k ? static_cast<int64_t>(__builtin_amdgcn_readlane(rv, j)) * H : 0;
    wts[j] = j < k ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wv), j)) : 0.f;
  }
  constexpr int kWords = YF == MOE_BF16 ? 1 : 2;  // 16-byte words per 8 values
  for (int c = threadIdx.x; c < nvec; c += 256) {
    // all k loads in flight before the first product
    u32x4_t raw[kMaxK][kWords];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < k) {
#pragma unroll
        for (int q = 0; q < kWords; ++q)
          raw[j][q] = YF == MOE_BF16
              ? *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(y) + rows[j] + c * 8)
              : reinterpret_cast<const u32x4_t*>(static_cast<const float*>(y) + rows[j] + c * 8)[q];
      }
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < k) {
        float v[8];
        if (YF == MOE_BF16) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(raw[j][0][i] << 16);
            v[2 * i + 1] = __uint_as_float(raw[j][0][i] & 0xFFFF0000u);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[i] = __uint_as_float(raw[j][0][i]);
            v[4 + i] = __uint_as_float(raw[j][kWords - 1][i]);
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(wts[j], v[i], acc[i]);
      }
    if (shared) {
      float v[8];
      load8<YF>(shared, static_cast<int64_t>(t) * H + c * 8, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    const int64_t o = static_cast<int64_t>(t) * H + c * 8;
    if (OF == MOE_BF16) {
      *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(out) + o) =
          u32x4_t{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                  pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
    } else {
      f32x4_t* p = reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + o);
      p[0] = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
      p[1] = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
    }
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_combine(const void* y, int y_fmt, const int32_t* row_map, const float* topk_w,
                           const void* shared, int T, int k, int H, void* out, int out_fmt,
                           hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(T >= 0 && k >= 1 && k <= kMaxK && H > 0 && H % 8 == 0, MOE_ERR_INVALID_ARG,
              "moe_combine: need T >= 0, 1 <= k <= 16, H a positive multiple of 8");
  MOE_REQUIRE((y_fmt == MOE_F32 || y_fmt == MOE_BF16) && (out_fmt == MOE_F32 || out_fmt == MOE_BF16),
              MOE_ERR_UNSUPPORTED, "moe_combine: formats must be MOE_F32 or MOE_BF16");
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(y && row_map && topk_w && out, MOE_ERR_INVALID_ARG, "moe_combine: null pointer");
  MOE_REQUIRE(aligned16(y) && aligned16(out) && (!shared || aligned16(shared)), MOE_ERR_ALIGNMENT,
              "moe_combine: y, shared and out must be 16-byte aligned");
  auto launch = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(T), dim3(256), 0, stream, y, row_map, topk_w, shared, T, k, H, out);
  };
  if (y_fmt == MOE_BF16) {
    if (out_fmt == MOE_BF16) launch(combine_kernel<MOE_BF16, MOE_BF16>);
    else launch(combine_kernel<MOE_BF16, MOE_F32>);
  } else {
    if (out_fmt == MOE_BF16) launch(combine_kernel<MOE_F32, MOE_BF16>);
    else launch(combine_kernel<MOE_F32, MOE_F32>);
  }
  return check_launch("moe_combine");
}

// Summing un-permute for the backward: dx[t] = sum_j dx_perm[row_map[t, j]]
// (the combine with unit weights and no shared row).
extern "C" int moe_unpermute(const void* dx_perm, int fmt, const int32_t* row_map, int T, int k,
                             int H, void* dx, int out_fmt, hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(T >= 0 && k >= 1 && k <= kMaxK && H > 0 && H % 8 == 0, MOE_ERR_INVALID_ARG,
              "moe_unpermute: need T >= 0, 1 <= k <= 16, H a positive multiple of 8");
  MOE_REQUIRE((fmt == MOE_F32 || fmt == MOE_BF16) && (out_fmt == MOE_F32 || out_fmt == MOE_BF16),
              MOE_ERR_UNSUPPORTED, "moe_unpermute: formats must be MOE_F32 or MOE_BF16");
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(dx_perm && row_map && dx, MOE_ERR_INVALID_ARG, "moe_unpermute: null pointer");
  MOE_REQUIRE(aligned16(dx_perm) && aligned16(dx), MOE_ERR_ALIGNMENT,
              "moe_unpermute: dx_perm and dx must be 16-byte aligned");
  const float* none = nullptr;
  auto launch = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(T), dim3(256), 0, stream, dx_perm, row_map, none, nullptr, T, k, H, dx);
  };
  if (fmt == MOE_BF16) {
    if (out_fmt == MOE_BF16) launch(combine_kernel<MOE_BF16, MOE_BF16>);
    else launch(combine_kernel<MOE_BF16, MOE_F32>);
  } else {
    if (out_fmt == MOE_BF16) launch(combine_kernel<MOE_F32, MOE_BF16>);
    else launch(combine_kernel<MOE_F32, MOE_F32>);
  }
  return check_launch("moe_unpermute");
}
