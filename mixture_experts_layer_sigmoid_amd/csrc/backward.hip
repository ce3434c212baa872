// Backward of the routed expert path: combine backward, segment-transposed
// MX quantization of the backward GEMM operands, and the C entry points of
// the backward grouped GEMMs (fc2 data gradient fused with the SwiGLU
// backward, fc1 data gradient, weight gradients).
//
// Page "[PyTorch] DeepSeekV3Layer: full MoE transformer layer (MLA +
// DeepSeek MoE)", Performance section, "Where the time goes" table: the
// fused grouped MLP runs "dGLU bwd" and "wgrad" in MXFP8, and the local
// permute runs its reduce in the backward too. Readings where the page is
// silent: routing weights are constants; quantizers pass gradients straight
// through; every backward GEMM operand is MX quantized along that GEMM's
// contraction axis (weights from a second, transposed quantization of the
// same masters; activations along the rows of each expert segment, in
// blocks of 32 rows of the segment padded to a multiple of 32).
#include "common.h"
#include "mx_codec.h"

#include <algorithm>
#include <type_traits>

namespace moe {
namespace {

constexpr int kMaxE = 1024;

template <int DF>
__device__ __forceinline__ void load_row8(const void* base, int64_t off, float* v) {
  if (DF == MOE_BF16) {
    const u32x4_t q = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(q[i] << 16);
      v[2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
    }
  } else {
    load8_f32(static_cast<const float*>(base) + off, v);
  }
}

// Routing weight of expert-major row r (0 for a padding row): the slot j of
// token src_row[r] whose row_map entry is r.
__device__ __forceinline__ float row_weight(const int32_t* row_map, const float* w, int t, int k,
                                            int64_t r) {
  float wj = 0.f;
  if (t >= 0)
    for (int j = 0; j < k; ++j)
      if (row_map[static_cast<int64_t>(t) * k + j] == r) wj = w[static_cast<int64_t>(t) * k + j];
  return wj;
}

// dy[r] = w[t, j] * dout[t] for the row r = row_map[t, j], formed in fp32;
// padding rows (src_row -1) are zero. One workgroup per row. Plain output
// (OF = MOE_F32 / MOE_BF16): 8 columns per thread. MX output: one 32-column
// block per thread, encoded from the fp32 products (no intermediate
// rounding), codes and one scale byte per block.
template <int DF, int OF>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const void* __restrict__ dout,
                                                          const int32_t* __restrict__ row_map,
                                                          const int32_t* __restrict__ src_row,
                                                          const float* __restrict__ w, int k, int H,
                                                          int64_t rows, void* __restrict__ dy,
                                                          uint8_t* __restrict__ dy_scales,
                                                          float* __restrict__ row_w) {
  constexpr bool kMx = OF == MOE_MXFP8_E4M3 || OF == MOE_MXFP4_E2M1;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const int t = src_row[r];
    const float wj = row_weight(row_map, w, t, k, r);
    if (row_w && threadIdx.x == 0) row_w[r] = wj;
    if constexpr (kMx) {
      constexpr bool fp4 = OF == MOE_MXFP4_E2M1;
      for (int b = threadIdx.x; b < H / 32; b += 256) {
        float v[32];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (t >= 0) {
            load_row8<DF>(dout, static_cast<int64_t>(t) * H + b * 32 + q * 8, v + q * 8);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[q * 8 + i] *= wj;
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[q * 8 + i] = 0.f;
          }
        }
        uint32_t words[8];
        const uint32_t sb = mx_encode_block<fp4>(v, words);
        uint8_t* o = static_cast<uint8_t*>(dy) + r * (fp4 ? H / 2 : H) + b * (fp4 ? 16 : 32);
        reinterpret_cast<u32x4_t*>(o)[0] = u32x4_t{words[0], words[1], words[2], words[3]};
        if (!fp4) reinterpret_cast<u32x4_t*>(o)[1] = u32x4_t{words[4], words[5], words[6], words[7]};
        dy_scales[r * (H / 32) + b] = static_cast<uint8_t>(sb);
      }
    } else {
      for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
        float v[8];
        if (t >= 0) {
          load_row8<DF>(dout, static_cast<int64_t>(t) * H + c, v);
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] *= wj;
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = 0.f;
        }
        if (OF == MOE_BF16) {
          *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(dy) + r * H + c) =
              u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                      pack_bf16x2(v[6], v[7])};
        } else {
          store8_f32(static_cast<float*>(dy) + r * H + c, v);
        }
      }
    }
  }
}

enum { SEG_ROWS = 0, SEG_GATHER = 1, SEG_SWIGLU = 2 };

// K-major MX quantization of row segments: codes[c, kofs[e] + i] for the
// segment's rows i (blocks of 32 rows), each segment padded with zeros to a
// multiple of `pad` columns; scales [c, kstride/32]. Input rows r
// (segments [offsets[e], offsets[e+1])) of C columns:
//   SEG_ROWS:   in[r, c], zero where src_row[r] < 0
//   SEG_GATHER: in[src_row[r], c] (token rows), zero where src_row < 0
//   SEG_SWIGLU: silu(in[r, c]) * in[r, C + c] (in is [rows, 2C])
// with an optional fp32 row_scale[r]. offsets == nullptr means one segment
// [0, rows); src_row == nullptr means every row is live. Used by
// moe_quantize_mx along axis 1 (one segment, pad 32).
template <int IN>
__device__ __forceinline__ float ld_in(const void* in, int64_t i) {
  if (IN == MOE_BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(in)[i]);
  return static_cast<const float*>(in)[i];
}

template <int MODE, bool FP4, int IN>
__global__ __launch_bounds__(256) void quantize_kmajor_kernel(
    const void* __restrict__ in, const int32_t* __restrict__ src_row,
    const int32_t* __restrict__ offsets, const float* __restrict__ row_scale, int E, int64_t rows,
    int C, int64_t kstride, int pad, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    int32_t* __restrict__ kofs_out) {
  __shared__ int32_t s_kofs[kMaxE + 1];
  __shared__ int32_t part[256];
  const int tid = threadIdx.x;
  {
    const int per = (E + 255) / 256;
    const int lo = tid * per, hi = min(E, lo + per);
    int s = 0;
    for (int e = lo; e < hi; ++e) {
      const int seg = offsets ? offsets[e + 1] - offsets[e] : static_cast<int>(rows);
      s_kofs[e + 1] = (seg + pad - 1) / pad * pad;
      s += s_kofs[e + 1];
    }
    part[tid] = s;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
      const int v = tid >= d ? part[tid - d] : 0;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    int run = tid > 0 ? part[tid - 1] : 0;
    for (int e = lo; e < hi; ++e) {
      run += s_kofs[e + 1];
      s_kofs[e + 1] = run;
    }
    if (tid == 0) s_kofs[0] = 0;
    __syncthreads();
  }
  if (blockIdx.x == 0 && kofs_out)
    for (int e = tid; e <= E; e += 256) kofs_out[e] = s_kofs[e];
  const int kblocks = s_kofs[E] / 32;
  const int cgroups = (C + 255) / 256;
  for (int64_t wi = blockIdx.x; wi < static_cast<int64_t>(kblocks) * cgroups; wi += gridDim.x) {
    const int kb = static_cast<int>(wi / cgroups);
    const int c = static_cast<int>(wi % cgroups) * 256 + tid;
    if (c >= C) continue;
    // the segment holding output columns [32kb, 32kb+32)
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_kofs[mid] <= kb * 32) lo = mid;
      else hi = mid;
    }
    const int e = lo;
    const int local = kb * 32 - s_kofs[e];
    const int64_t seg_lo = offsets ? offsets[e] : 0;
    const int seg = offsets ? offsets[e + 1] - offsets[e] : static_cast<int>(rows);
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      float x = 0.f;
      if (local + i < seg) {
        const int64_t r = seg_lo + local + i;
        const int src = src_row ? src_row[r] : static_cast<int>(r);
        if (src >= 0) {
          if (MODE == SEG_ROWS) {
            x = ld_in<IN>(in, r * C + c);
          } else if (MODE == SEG_GATHER) {
            x = ld_in<IN>(in, static_cast<int64_t>(src) * C + c);
          } else {
            const float g = ld_in<IN>(in, r * 2 * C + c);
            const float u = ld_in<IN>(in, r * 2 * C + C + c);
            x = g * (1.f / (1.f + expf(-g))) * u;
          }
          if (row_scale) x *= row_scale[r];
        }
      }
      v[i] = x;
    }
    uint32_t words[8];
    const uint32_t sb = mx_encode_block<FP4>(v, words);
    if (FP4) {
      *reinterpret_cast<u32x4_t*>(codes + static_cast<int64_t>(c) * (kstride / 2) + kb * 16) =
          u32x4_t{words[0], words[1], words[2], words[3]};
    } else {
      u32x4_t* o = reinterpret_cast<u32x4_t*>(codes + static_cast<int64_t>(c) * kstride + kb * 32);
      o[0] = u32x4_t{words[0], words[1], words[2], words[3]};
      o[1] = u32x4_t{words[4], words[5], words[6], words[7]};
    }
    scales[static_cast<int64_t>(c) * (kstride / 32) + kb] = static_cast<uint8_t>(sb);
  }
}


// Stage-major MX quantization of the weight-gradient operands. The K axis
// (the rows of the expert segments, each padded to a multiple of 128) is cut
// into stages of 128; stage g holds K columns [128g, 128g + 128) of every
// channel c as 128 contiguous E4M3 bytes:
//   codes  [kstride/128][C][128],  scales [kstride/128][C][4]
// so one 128-channel block of one stage is a contiguous 16 KB tile (what a
// weight-gradient tile loads per stage). A workgroup item is (stage, 64
// channels): it reads the stage's 128 rows x 64 channels (row-contiguous),
// forms the fp32 values in an LDS tile, encodes 4 blocks of 32 rows per
// channel and writes 64 x 128 contiguous code bytes and 64 x 4 scale bytes.
constexpr int kSegCols = 64;
template <int MODE, int IN>
__global__ __launch_bounds__(256) void quantize_stages_kernel(
    const void* __restrict__ in, const int32_t* __restrict__ src_row,
    const int32_t* __restrict__ offsets, const float* __restrict__ row_scale, int E, int C,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int32_t* __restrict__ kofs_out) {
  __shared__ int32_t s_kofs[kMaxE + 1];
  __shared__ int32_t part[256];
  __shared__ float tile[128][kSegCols + 1];
  __shared__ __attribute__((aligned(16))) uint8_t ocodes[kSegCols * 128];
  __shared__ __attribute__((aligned(16))) uint8_t oscale[kSegCols * 4];
  const int tid = threadIdx.x;
  {
    const int per = (E + 255) / 256;
    const int lo = min(E, tid * per), hi = min(E, lo + per);
    int s = 0;
    for (int e = lo; e < hi; ++e) {
      const int seg = offsets[e + 1] - offsets[e];
      s_kofs[e + 1] = (seg + 127) / 128 * 128;
      s += s_kofs[e + 1];
    }
    part[tid] = s;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
      const int v = tid >= d ? part[tid - d] : 0;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    int run = tid > 0 ? part[tid - 1] : 0;
    for (int e = lo; e < hi; ++e) {
      run += s_kofs[e + 1];
      s_kofs[e + 1] = run;
    }
    if (tid == 0) s_kofs[0] = 0;
    __syncthreads();
  }
  if (blockIdx.x == 0 && kofs_out)
    for (int e = tid; e <= E; e += 256) kofs_out[e] = s_kofs[e];
  const int nstage = s_kofs[E] / 128;
  const int ncb = (C + kSegCols - 1) / kSegCols;
  const int64_t n_items = static_cast<int64_t>(nstage) * ncb;
  // ---- input of one item: 128 rows x 64 channels; unit = (row, 8 channels),
  // 4 units per thread; raw 16-byte words held in registers so the next
  // item's loads are in flight while this one is encoded ----
  constexpr int kW = (IN == MOE_BF16 ? 1 : 2) * (MODE == SEG_SWIGLU ? 2 : 1);
  u32x4_t raw[4][kW];
  float rsc[4];
  bool ok[4];
  int cur_g = 0, cur_c0 = 0;
  auto load_item = [&](int64_t item) {
    const int g = static_cast<int>(item / ncb);
    const int c0 = static_cast<int>(item - static_cast<int64_t>(g) * ncb) * kSegCols;
    cur_g = g;
    cur_c0 = c0;
    int lo = 0, hi = E;  // the segment holding K columns [128g, 128g + 128)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_kofs[mid] <= g * 128) lo = mid;
      else hi = mid;
    }
    const int local0 = g * 128 - s_kofs[lo];
    const int seg_lo = offsets[lo];
    const int seg = offsets[lo + 1] - seg_lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = tid + 256 * i;
      const int r = u >> 3, c = c0 + (u & 7) * 8;
      ok[i] = false;
      rsc[i] = 1.f;
      if (local0 + r < seg && c < C) {
        const int64_t row = seg_lo + local0 + r;
        const int src = src_row[row];
        if (src >= 0) {
          ok[i] = true;
          const int64_t srow = MODE == SEG_GATHER ? src : row;
          const int64_t stride = MODE == SEG_SWIGLU ? 2ll * C : C;
          const int64_t off = srow * stride + c;  // elements
#pragma unroll
          for (int w = 0; w < kW; ++w) {
            // bf16: one word of 8 values (+ the up half for SwiGLU);
            // fp32: two words of 4 values each (x2 for SwiGLU)
            const int half = IN == MOE_BF16 ? w : w / 2;         // 0 gate / plain, 1 up
            const int part = IN == MOE_BF16 ? 0 : w % 2;
            const int64_t e0 = off + (MODE == SEG_SWIGLU ? half * C : 0) + 4 * part;
            raw[i][w] = IN == MOE_BF16
                ? *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(in) + e0)
                : *reinterpret_cast<const u32x4_t*>(static_cast<const float*>(in) + e0);
          }
          if (row_scale) rsc[i] = row_scale[row];
        }
      }
    }
  };
  auto values = [&](int i, float* v) {  // unit i's 8 fp32 values
    float a[8], b[8];
    auto unpack = [&](int first, float* o) {
      if constexpr (IN == MOE_BF16) {
        const u32x4_t q = raw[i][first];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          o[2 * t] = __uint_as_float(q[t] << 16);
          o[2 * t + 1] = __uint_as_float(q[t] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          o[t] = __uint_as_float(raw[i][first][t]);
          o[4 + t] = __uint_as_float(raw[i][first + 1][t]);
        }
      }
    };
    if (!ok[i]) {
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = 0.f;
      return;
    }
    unpack(0, a);
    if constexpr (MODE == SEG_SWIGLU) {
      unpack(IN == MOE_BF16 ? 1 : 2, b);
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = a[q] * (1.f / (1.f + expf(-a[q]))) * b[q];
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = a[q];
    }
    if (row_scale) {
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] *= rsc[i];
    }
  };
  int64_t item = blockIdx.x;
  if (item < n_items) load_item(item);
  for (; item < n_items; item += gridDim.x) {
    const int g = cur_g, c0 = cur_c0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = tid + 256 * i;
      float v[8];
      values(i, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) tile[u >> 3][(u & 7) * 8 + q] = v[q];
    }
    __syncthreads();
    if (item + gridDim.x < n_items) load_item(item + gridDim.x);
    // ---- encode: thread -> (channel t % 64, block of 32 rows t / 64) ----
    {
      const int c = tid & 63, b = tid >> 6;
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = tile[32 * b + i][c];
      uint32_t words[8];
      const uint32_t sb = mx_encode_block<false>(v, words);
      u32x4_t* o = reinterpret_cast<u32x4_t*>(ocodes + c * 128 + 32 * b);
      o[0] = u32x4_t{words[0], words[1], words[2], words[3]};
      o[1] = u32x4_t{words[4], words[5], words[6], words[7]};
      oscale[c * 4 + b] = static_cast<uint8_t>(sb);
    }
    __syncthreads();
    // ---- 64 channel rows of 128 code bytes, contiguous in the output ----
    const int64_t obase = static_cast<int64_t>(g) * C + c0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 256 * i;  // 16-byte chunk: channel q / 8, part q % 8
      if (c0 + (q >> 3) < C)
        *reinterpret_cast<u32x4_t*>(codes + (obase + (q >> 3)) * 128 + (q & 7) * 16) =
            *reinterpret_cast<const u32x4_t*>(ocodes + q * 16);
    }
    if (tid < kSegCols && c0 + tid < C)
      *reinterpret_cast<uint32_t*>(scales + (obase + tid) * 4) =
          *reinterpret_cast<const uint32_t*>(oscale + tid * 4);
    __syncthreads();
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_combine_bwd(const void* dout, int dout_fmt, const int32_t* row_map,
                               const int32_t* src_row, const float* topk_w, int T, int k, int H,
                               int64_t rows, void* dy, int dy_fmt, uint8_t* dy_scales,
                               float* row_w, hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(T >= 0 && k >= 1 && H > 0 && H % 8 == 0 && rows >= 0, MOE_ERR_INVALID_ARG,
              "moe_combine_bwd: need T >= 0, k >= 1, H a positive multiple of 8, rows >= 0");
  MOE_REQUIRE(dout_fmt == MOE_BF16 || dout_fmt == MOE_F32, MOE_ERR_UNSUPPORTED,
              "moe_combine_bwd: dout_fmt must be MOE_BF16 or MOE_F32");
  const bool mx = dy_fmt == MOE_MXFP8_E4M3 || dy_fmt == MOE_MXFP4_E2M1;
  MOE_REQUIRE(mx || dy_fmt == MOE_BF16 || dy_fmt == MOE_F32, MOE_ERR_UNSUPPORTED,
              "moe_combine_bwd: dy_fmt must be MOE_F32, MOE_BF16 or an MX format");
  MOE_REQUIRE(!mx || H % 32 == 0, MOE_ERR_INVALID_ARG, "moe_combine_bwd: MX dy needs H % 32 == 0");
  if (rows == 0) return MOE_OK;
  MOE_REQUIRE(dy && src_row && (!mx || dy_scales) && (T == 0 || (dout && row_map && topk_w)),
              MOE_ERR_INVALID_ARG, "moe_combine_bwd: null pointer");
  MOE_REQUIRE(aligned16(dy) && (!dout || aligned16(dout)), MOE_ERR_ALIGNMENT,
              "moe_combine_bwd: dout and dy must be 16-byte aligned");
  const unsigned grid = static_cast<unsigned>(std::min<int64_t>(rows, 16384));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, stream, dout, row_map, src_row, topk_w, k, H,
                       rows, dy, dy_scales, row_w);
  };
  auto by_out = [&](auto df) {
    constexpr int DF = decltype(df)::value;
    switch (dy_fmt) {
      case MOE_F32: go(combine_bwd_kernel<DF, MOE_F32>); break;
      case MOE_BF16: go(combine_bwd_kernel<DF, MOE_BF16>); break;
      case MOE_MXFP8_E4M3: go(combine_bwd_kernel<DF, MOE_MXFP8_E4M3>); break;
      default: go(combine_bwd_kernel<DF, MOE_MXFP4_E2M1>); break;
    }
  };
  if (dout_fmt == MOE_BF16) by_out(std::integral_constant<int, MOE_BF16>{});
  else by_out(std::integral_constant<int, MOE_F32>{});
  return check_launch("moe_combine_bwd");
}

extern "C" int64_t moe_segments_kstride(int64_t rows, int E) {
  if (rows < 0 || E < 1) return -1;
  return (rows + static_cast<int64_t>(E) * 127 + 127) / 128 * 128;
}

extern "C" int moe_quantize_mx_segments(const void* in, int in_fmt, int mode,
                                        const int32_t* src_row, const int32_t* offsets,
                                        const float* row_scale, int E, int64_t rows, int C,
                                        int64_t kstride, int out_fmt, uint8_t* codes,
                                        uint8_t* scales, int32_t* kofs, hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(E >= 1 && E <= kMaxE && C > 0 && C % 8 == 0 && rows >= 0, MOE_ERR_INVALID_ARG,
              "moe_quantize_mx_segments: need 1 <= E <= 1024, C a positive multiple of 8, rows >= 0");
  MOE_REQUIRE(mode >= SEG_ROWS && mode <= SEG_SWIGLU, MOE_ERR_INVALID_ARG,
              "moe_quantize_mx_segments: mode must be 0 (rows), 1 (gather) or 2 (swiglu)");
  MOE_REQUIRE(in_fmt == MOE_BF16 || in_fmt == MOE_F32, MOE_ERR_UNSUPPORTED,
              "moe_quantize_mx_segments: in_fmt must be MOE_BF16 or MOE_F32");
  MOE_REQUIRE(out_fmt == MOE_MXFP8_E4M3, MOE_ERR_UNSUPPORTED,
              "moe_quantize_mx_segments: out_fmt must be MOE_MXFP8_E4M3");
  MOE_REQUIRE(kstride >= moe_segments_kstride(rows, E) && kstride % 128 == 0, MOE_ERR_INVALID_ARG,
              "moe_quantize_mx_segments: kstride below moe_segments_kstride(rows, E) or not a "
              "multiple of 128");
  MOE_REQUIRE(in && src_row && offsets && codes && scales && kofs, MOE_ERR_INVALID_ARG,
              "moe_quantize_mx_segments: null pointer");
  MOE_REQUIRE(aligned16(codes) && aligned16(in) && (reinterpret_cast<uintptr_t>(scales) & 3u) == 0,
              MOE_ERR_ALIGNMENT,
              "moe_quantize_mx_segments: in and codes must be 16-byte, scales 4-byte aligned");
  const int64_t work = (kstride / 128) * ((C + kSegCols - 1) / kSegCols);
  const unsigned grid = static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>(work, 1536)));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, stream, in, src_row, offsets, row_scale, E,
                       C, codes, scales, kofs);
  };
  auto by_mode = [&](auto in_c) {
    constexpr int IN = decltype(in_c)::value;
    if (mode == SEG_ROWS) go(quantize_stages_kernel<SEG_ROWS, IN>);
    else if (mode == SEG_GATHER) go(quantize_stages_kernel<SEG_GATHER, IN>);
    else go(quantize_stages_kernel<SEG_SWIGLU, IN>);
  };
  if (in_fmt == MOE_BF16) by_mode(std::integral_constant<int, MOE_BF16>{});
  else by_mode(std::integral_constant<int, MOE_F32>{});
  return check_launch("moe_quantize_mx_segments");
}

namespace moe {
// moe_quantize_mx with axis 1: [rows, K] -> K-major codes [K, rows] (E2M1:
// [K, rows/2]) and scales [K, rows/32], blocks of 32 consecutive rows.
int quantize_mx_columns(const void* in, int64_t rows, int K, int out_fmt, uint8_t* codes,
                        uint8_t* scales, hipStream_t stream) {
  const int64_t work = (rows / 32) * ((K + 255) / 256);
  const unsigned grid = static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>(work, 16384)));
  if (out_fmt == MOE_MXFP4_E2M1)
    hipLaunchKernelGGL((quantize_kmajor_kernel<SEG_ROWS, true, MOE_BF16>), dim3(grid), dim3(256), 0,
                       stream, in, nullptr, nullptr, nullptr, 1, rows, K, rows, 32, codes, scales,
                       nullptr);
  else
    hipLaunchKernelGGL((quantize_kmajor_kernel<SEG_ROWS, false, MOE_BF16>), dim3(grid), dim3(256), 0,
                       stream, in, nullptr, nullptr, nullptr, 1, rows, K, rows, 32, codes, scales,
                       nullptr);
  return check_launch("moe_quantize_mx");
}
}  // namespace moe
