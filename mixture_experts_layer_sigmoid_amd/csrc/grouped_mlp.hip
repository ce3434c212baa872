// Entry points of the grouped expert MLP: routed fc1 + SwiGLU (+ MX
// quantization of h), fc2, the fused routed + shared expert launches, the
// whole forward (moe_grouped_mlp_fwd) and the data-gradient GEMMs of the
// backward. Argument checks run here, on the host, before anything is
// enqueued; the GEMMs themselves are the packed-weight grouped kernel of
// expert_gemm.hip, except for fp32 layers, which use the plain kernels below
// (the tiny fp32 layer is launch-latency bound).
//
// Page "[PyTorch] DeepSeekV3Layer: full MoE transformer layer (MLA +
// DeepSeek MoE)": Description (experts as GroupedLinear -> ScaledSwiGLU ->
// GroupedLinear, fused into one grouped MLP; optional shared expert) and
// Performance section ("Where the time goes": fused grouped MLP, fc1+SwiGLU
// fwd, fc2 fwd and dGLU bwd, MXFP8). Page "Mistral Large 3 NVFP4 TRTLLM MoE
// support", Highlights: fc1's weight holds the w1 (gate) and w3 (up) halves;
// here rows [0, F) gate, [F, 2F) up.

#include "common.h"
#include "gemm_util.h"
#include "expert_gemm.h"

#include <algorithm>

namespace moe {
namespace {

constexpr int kMaxGroups = 1024;

// ---------------------------------------------------------------------------
// fp32 path (the small fp32 layer): plain FMA, one thread per output.
__global__ __launch_bounds__(256) void fc1_swiglu_f32_kernel(const float* __restrict__ a,
                                                             const int32_t* __restrict__ gather,
                                                             const float* __restrict__ w1,
                                                             const int32_t* __restrict__ offsets,
                                                             int E, int H, int F, int64_t rows,
                                                             float* __restrict__ h,
                                                             float* __restrict__ act_save) {
  const int64_t used = min(static_cast<int64_t>(offsets[E]), rows);
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < used * F; i += 256ll * gridDim.x) {
    const int64_t r = i / F;
    const int c = static_cast<int>(i % F);
    int lo = 0, hi = E;  // expert of row r: offsets[lo] <= r < offsets[lo+1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (offsets[mid] <= r) lo = mid;
      else hi = mid;
    }
    int64_t src = r;
    if (gather) src = gather[r];
    if (src < 0) {
      h[r * F + c] = 0.f;
      continue;
    }
    const float* x = a + src * H;
    const float* wg = w1 + (static_cast<int64_t>(lo) * 2 * F + c) * H;
    const float* wu = wg + static_cast<int64_t>(F) * H;
    float g = 0.f, u = 0.f;
    for (int k = 0; k < H; ++k) {
      g = fmaf(x[k], wg[k], g);
      u = fmaf(x[k], wu[k], u);
    }
    if (act_save) {
      act_save[r * 2 * F + c] = g;
      act_save[r * 2 * F + F + c] = u;
    }
    h[r * F + c] = silu_mul(g, u);
  }
}

__global__ __launch_bounds__(256) void fc2_f32_kernel(const float* __restrict__ h,
                                                      const float* __restrict__ w2,
                                                      const int32_t* __restrict__ offsets, int E,
                                                      int H, int F, int64_t rows,
                                                      float* __restrict__ y) {
  const int64_t used = min(static_cast<int64_t>(offsets[E]), rows);
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < used * H; i += 256ll * gridDim.x) {
    const int64_t r = i / H;
    const int c = static_cast<int>(i % H);
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (offsets[mid] <= r) lo = mid;
      else hi = mid;
    }
    const float* hr = h + r * F;
    const float* w = w2 + (static_cast<int64_t>(lo) * H + c) * F;
    float acc = 0.f;
    for (int k = 0; k < F; ++k) acc = fmaf(hr[k], w[k], acc);
    y[r * H + c] = acc;
  }
}

int elem_bits(int fmt) {
  switch (fmt) {
    case MOE_F32: return 32;
    case MOE_BF16: return 16;
    case MOE_MXFP8_E4M3: return 8;
    case MOE_MXFP4_E2M1: return 4;
    default: return 0;
  }
}

static size_t h_bytes_of(int64_t rows, int F, int fmt) {
  const size_t h = static_cast<size_t>(rows) * F * elem_bits(fmt) / 8;
  return (h + 255) & ~static_cast<size_t>(255);
}

static bool is_mx(int f) { return f == MOE_MXFP8_E4M3 || f == MOE_MXFP4_E2M1; }

// Shared argument checks of the grouped calls; `h_fmt` is the format of the
// SwiGLU output (the activation format of the layer), `y_fmt` that of y.
static int check_formats(const char* fn, int a_fmt, int w_fmt, int y_fmt, int H, int F) {
  const bool f32 = a_fmt == MOE_F32 && w_fmt == MOE_F32 && y_fmt == MOE_F32;
  const bool bf16 = a_fmt == MOE_BF16 && w_fmt == MOE_BF16 && y_fmt == MOE_BF16;
  const bool fp8 = a_fmt == MOE_MXFP8_E4M3 && w_fmt == MOE_MXFP8_E4M3 && y_fmt == MOE_BF16;
  const bool fp4 = a_fmt == MOE_MXFP4_E2M1 && w_fmt == MOE_MXFP4_E2M1 && y_fmt == MOE_BF16;
  std::string f(fn);
  MOE_REQUIRE(f32 || bf16 || fp8 || fp4, MOE_ERR_UNSUPPORTED,
              f + ": supported (a, w, y) formats are (F32,F32,F32), (BF16,BF16,BF16), "
                  "(MXFP8,MXFP8,BF16), (MXFP4,MXFP4,BF16)");
  if (bf16)
    MOE_REQUIRE(H % 128 == 0 && F % 64 == 0, MOE_ERR_INVALID_ARG,
                f + ": bf16 needs H % 128 == 0 and F % 64 == 0");
  if (fp8)
    MOE_REQUIRE(H % 128 == 0 && F % 128 == 0, MOE_ERR_INVALID_ARG,
                f + ": MXFP8 needs H % 128 == 0 and F % 128 == 0");
  if (fp4)
    MOE_REQUIRE(H % 256 == 0 && F % 256 == 0, MOE_ERR_INVALID_ARG,
                f + ": MXFP4 needs H % 256 == 0 and F % 256 == 0");
  return MOE_OK;
}

static bool scale_aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }

static int fc1_impl(const void* a, const uint8_t* a_scales, int a_fmt, const int32_t* src_row,
                    const void* w1, const uint8_t* w1_scales, const int32_t* offsets, int E, int H,
                    int F, int64_t rows, float* act_save, void* h, uint8_t* h_scales,
                    hipStream_t stream) {
  if (a_fmt == MOE_F32) {
    const int64_t g1 = std::min<int64_t>(65536, (rows * F + 255) / 256);
    hipLaunchKernelGGL(fc1_swiglu_f32_kernel, dim3(g1), dim3(256), 0, stream,
                       static_cast<const float*>(a), src_row, static_cast<const float*>(w1),
                       offsets, E, H, F, rows, static_cast<float*>(h),
                       static_cast<float*>(act_save));
    return check_launch("moe_grouped_fc1_swiglu");
  }
  return expert_gemm(0, a, a_scales, a_fmt, src_row, w1, w1_scales, offsets, E, 2 * F, H, rows,
                     F, h, h_scales, act_save, nullptr, nullptr, stream);
}

static int fc2_impl(const void* h, const uint8_t* h_scales, int h_fmt, const void* w2,
                    const uint8_t* w2_scales, const int32_t* offsets, int E, int H, int F,
                    int64_t rows, void* y, hipStream_t stream) {
  if (h_fmt == MOE_F32) {
    const int64_t g2 = std::min<int64_t>(65536, (rows * H + 255) / 256);
    hipLaunchKernelGGL(fc2_f32_kernel, dim3(g2), dim3(256), 0, stream,
                       static_cast<const float*>(h), static_cast<const float*>(w2), offsets, E, H,
                       F, rows, static_cast<float*>(y));
    return check_launch("moe_grouped_fc2");
  }
  return expert_gemm(1, h, h_scales, h_fmt, nullptr, w2, w2_scales, offsets, E, H, F, rows, 0, y,
                     nullptr, nullptr, nullptr, nullptr, stream);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_grouped_mlp_workspace(int E, int H, int F, int64_t rows, int a_fmt,
                                            int w_fmt) {
  (void)E;
  (void)H;
  (void)w_fmt;
  if (rows < 0 || F <= 0 || elem_bits(a_fmt) == 0) return 0;
  size_t sc = is_mx(a_fmt) ? static_cast<size_t>(rows) * (F / 32) : 0;
  sc = (sc + 255) & ~static_cast<size_t>(255);
  return h_bytes_of(rows, F, a_fmt) + sc;
}

extern "C" int moe_grouped_fc1_swiglu(const void* a, const uint8_t* a_scales, int a_fmt,
                                      const int32_t* src_row, const void* w1,
                                      const uint8_t* w1_scales, int w_fmt,
                                      const int32_t* offsets, int E, int H, int F, int64_t rows,
                                      float* act_save, void* h, uint8_t* h_scales,
                                      hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(E >= 1 && E <= kMaxGroups && H > 0 && F > 0 && rows >= 0, MOE_ERR_INVALID_ARG,
              "moe_grouped_fc1_swiglu: need 1 <= E <= 1024, H > 0, F > 0, rows >= 0");
  const int y_like = a_fmt == MOE_F32 ? MOE_F32 : MOE_BF16;
  int st = check_formats("moe_grouped_fc1_swiglu", a_fmt, w_fmt, y_like, H, F);
  if (st) return st;
  if (rows == 0) return MOE_OK;  // nothing to read or write; pointers may be null
  MOE_REQUIRE(offsets && w1 && h && (rows == 0 || a), MOE_ERR_INVALID_ARG,
              "moe_grouped_fc1_swiglu: null pointer");
  if (is_mx(a_fmt))
    MOE_REQUIRE(a_scales && w1_scales && h_scales, MOE_ERR_INVALID_ARG,
                "moe_grouped_fc1_swiglu: MX formats need a_scales, w1_scales and h_scales");
  MOE_REQUIRE(aligned16(a) && aligned16(w1) && aligned16(h) && (!act_save || aligned16(act_save)),
              MOE_ERR_ALIGNMENT, "moe_grouped_fc1_swiglu: tensors must be 16-byte aligned");
  if (is_mx(a_fmt))
    MOE_REQUIRE(scale_aligned(a_scales) && scale_aligned(w1_scales), MOE_ERR_ALIGNMENT,
                "moe_grouped_fc1_swiglu: scale arrays must be 4-byte aligned");
  if (rows == 0) return MOE_OK;
  return fc1_impl(a, a_scales, a_fmt, src_row, w1, w1_scales, offsets, E, H, F, rows, act_save, h,
                  h_scales, stream);
}

extern "C" int moe_grouped_fc2(const void* h, const uint8_t* h_scales, int h_fmt, const void* w2,
                               const uint8_t* w2_scales, int w_fmt, const int32_t* offsets, int E,
                               int H, int F, int64_t rows, void* y, int y_fmt,
                               hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(E >= 1 && E <= kMaxGroups && H > 0 && F > 0 && rows >= 0, MOE_ERR_INVALID_ARG,
              "moe_grouped_fc2: need 1 <= E <= 1024, H > 0, F > 0, rows >= 0");
  int st = check_formats("moe_grouped_fc2", h_fmt, w_fmt, y_fmt, H, F);
  if (st) return st;
  if (rows == 0) return MOE_OK;  // nothing to read or write; pointers may be null
  MOE_REQUIRE(offsets && w2 && (rows == 0 || (h && y)), MOE_ERR_INVALID_ARG,
              "moe_grouped_fc2: null pointer");
  if (is_mx(h_fmt))
    MOE_REQUIRE(h_scales && w2_scales, MOE_ERR_INVALID_ARG,
                "moe_grouped_fc2: MX formats need h_scales and w2_scales");
  MOE_REQUIRE(aligned16(h) && aligned16(w2) && aligned16(y), MOE_ERR_ALIGNMENT,
              "moe_grouped_fc2: tensors must be 16-byte aligned");
  if (is_mx(h_fmt))
    MOE_REQUIRE(scale_aligned(h_scales) && scale_aligned(w2_scales), MOE_ERR_ALIGNMENT,
                "moe_grouped_fc2: scale arrays must be 4-byte aligned");
  if (rows == 0) return MOE_OK;
  return fc2_impl(h, h_scales, h_fmt, w2, w2_scales, offsets, E, H, F, rows, y, stream);
}

// fc1 / fc2 of the routed experts and an always-on dense expert (the
// shared expert) in one launch each: the dense expert's T rows follow the
// routed rows in h and y. Its tiles are spread through the tile list, so
// its matrix work runs beside the routed weight stream.
extern "C" int moe_grouped_fc1_swiglu_dense(const void* a, const uint8_t* a_scales, int a_fmt,
                                            const int32_t* src_row, const void* w1,
                                            const uint8_t* w1_scales, int w_fmt,
                                            const int32_t* offsets, int E, int H, int F,
                                            int64_t rows, float* act_save, void* h,
                                            uint8_t* h_scales, const void* w1d,
                                            const uint8_t* w1d_scales, int T,
                                            hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(E >= 1 && E <= kMaxGroups && H > 0 && F > 0 && rows >= 0 && T >= 0 &&
                  rows + T < (int64_t{1} << 31),
              MOE_ERR_INVALID_ARG,
              "moe_grouped_fc1_swiglu_dense: need 1 <= E <= 1024, H, F > 0, rows, T >= 0");
  MOE_REQUIRE(a_fmt != MOE_F32, MOE_ERR_UNSUPPORTED,
              "moe_grouped_fc1_swiglu_dense: fp32 layers run the shared expert separately");
  int st = check_formats("moe_grouped_fc1_swiglu_dense", a_fmt, w_fmt, MOE_BF16, H, F);
  if (st) return st;
  if (rows + T == 0) return MOE_OK;
  MOE_REQUIRE(offsets && w1 && w1d && h && (rows + T == 0 || a) && (rows == 0 || src_row),
              MOE_ERR_INVALID_ARG, "moe_grouped_fc1_swiglu_dense: null pointer");
  if (is_mx(a_fmt))
    MOE_REQUIRE(a_scales && w1_scales && w1d_scales && h_scales, MOE_ERR_INVALID_ARG,
                "moe_grouped_fc1_swiglu_dense: MX formats need a_scales, w1_scales, w1d_scales "
                "and h_scales");
  MOE_REQUIRE(aligned16(a) && aligned16(w1) && aligned16(w1d) && aligned16(h) &&
                  (!act_save || aligned16(act_save)),
              MOE_ERR_ALIGNMENT, "moe_grouped_fc1_swiglu_dense: tensors must be 16-byte aligned");
  if (is_mx(a_fmt))
    MOE_REQUIRE(scale_aligned(a_scales) && scale_aligned(w1_scales) && scale_aligned(w1d_scales),
                MOE_ERR_ALIGNMENT, "moe_grouped_fc1_swiglu_dense: scale arrays must be 4-byte aligned");
  if (rows + T == 0) return MOE_OK;
  const DenseExpert d{w1d, w1d_scales, T, static_cast<int>(rows), 0};
  return expert_gemm(0, a, a_scales, a_fmt, src_row, w1, w1_scales, offsets, E, 2 * F, H, rows,
                     F, h, h_scales, act_save, nullptr, nullptr, stream, &d);
}

extern "C" int moe_grouped_fc2_dense(const void* h, const uint8_t* h_scales, int h_fmt,
                                     const void* w2, const uint8_t* w2_scales, int w_fmt,
                                     const int32_t* offsets, int E, int H, int F, int64_t rows,
                                     void* y, int y_fmt, const void* w2d,
                                     const uint8_t* w2d_scales, int T, hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(E >= 1 && E <= kMaxGroups && H > 0 && F > 0 && rows >= 0 && T >= 0 &&
                  rows + T < (int64_t{1} << 31),
              MOE_ERR_INVALID_ARG, "moe_grouped_fc2_dense: need 1 <= E <= 1024, H, F > 0, rows, T >= 0");
  MOE_REQUIRE(h_fmt != MOE_F32, MOE_ERR_UNSUPPORTED,
              "moe_grouped_fc2_dense: fp32 layers run the shared expert separately");
  int st = check_formats("moe_grouped_fc2_dense", h_fmt, w_fmt, y_fmt, H, F);
  if (st) return st;
  if (rows + T == 0) return MOE_OK;
  MOE_REQUIRE(offsets && w2 && w2d && (rows + T == 0 || (h && y)), MOE_ERR_INVALID_ARG,
              "moe_grouped_fc2_dense: null pointer");
  if (is_mx(h_fmt))
    MOE_REQUIRE(h_scales && w2_scales && w2d_scales, MOE_ERR_INVALID_ARG,
                "moe_grouped_fc2_dense: MX formats need h_scales, w2_scales and w2d_scales");
  MOE_REQUIRE(aligned16(h) && aligned16(w2) && aligned16(w2d) && aligned16(y), MOE_ERR_ALIGNMENT,
              "moe_grouped_fc2_dense: tensors must be 16-byte aligned");
  if (is_mx(h_fmt))
    MOE_REQUIRE(scale_aligned(h_scales) && scale_aligned(w2_scales) && scale_aligned(w2d_scales),
                MOE_ERR_ALIGNMENT, "moe_grouped_fc2_dense: scale arrays must be 4-byte aligned");
  if (rows + T == 0) return MOE_OK;
  const DenseExpert d{w2d, w2d_scales, T, static_cast<int>(rows), static_cast<int>(rows)};
  return expert_gemm(1, h, h_scales, h_fmt, nullptr, w2, w2_scales, offsets, E, H, F, rows, 0, y,
                     nullptr, nullptr, nullptr, nullptr, stream, &d);
}

extern "C" int moe_grouped_mlp_fwd(const void* a, const uint8_t* a_scales, int a_fmt,
                                   const int32_t* src_row, const void* w1,
                                   const uint8_t* w1_scales, const void* w2,
                                   const uint8_t* w2_scales, int w_fmt, const int32_t* offsets,
                                   int E, int H, int F, int64_t rows, float* act_save, void* y,
                                   int y_fmt, void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(E >= 1 && E <= kMaxGroups && H > 0 && F > 0 && rows >= 0, MOE_ERR_INVALID_ARG,
              "moe_grouped_mlp_fwd: need 1 <= E <= 1024, H > 0, F > 0, rows >= 0");
  int st = check_formats("moe_grouped_mlp_fwd", a_fmt, w_fmt, y_fmt, H, F);
  if (st) return st;
  MOE_REQUIRE(offsets && w1 && w2 && y && (rows == 0 || a), MOE_ERR_INVALID_ARG,
              "moe_grouped_mlp_fwd: null pointer");
  const bool mx = is_mx(a_fmt);
  if (mx)
    MOE_REQUIRE(a_scales && w1_scales && w2_scales, MOE_ERR_INVALID_ARG,
                "moe_grouped_mlp_fwd: MX formats need a_scales, w1_scales and w2_scales");
  MOE_REQUIRE(aligned16(a) && aligned16(w1) && aligned16(w2) && aligned16(y) &&
                  (!act_save || aligned16(act_save)),
              MOE_ERR_ALIGNMENT, "moe_grouped_mlp_fwd: tensors must be 16-byte aligned");
  if (mx)
    MOE_REQUIRE(scale_aligned(a_scales) && scale_aligned(w1_scales) && scale_aligned(w2_scales),
                MOE_ERR_ALIGNMENT, "moe_grouped_mlp_fwd: scale arrays must be 4-byte aligned");
  const size_t need = moe_grouped_mlp_workspace(E, H, F, rows, a_fmt, w_fmt);
  MOE_REQUIRE(ws && ws_bytes >= need, MOE_ERR_WORKSPACE, "moe_grouped_mlp_fwd: workspace too small");
  if (rows == 0) return MOE_OK;
  uint8_t* h = static_cast<uint8_t*>(ws);
  uint8_t* h_sc = mx ? h + h_bytes_of(rows, F, a_fmt) : nullptr;
  st = fc1_impl(a, a_scales, a_fmt, src_row, w1, w1_scales, offsets, E, H, F, rows, act_save, h,
                h_sc, stream);
  if (st) return st;
  return fc2_impl(h, h_sc, a_fmt, w2, w2_scales, offsets, E, H, F, rows, y, stream);
}

// ---------------------------------------------------------------------------
// Backward grouped GEMMs (page "[PyTorch] DeepSeekV3Layer: full MoE
// transformer layer (MLA + DeepSeek MoE)", Performance section, "Where the
// time goes": dGLU bwd of the fused grouped MLP; its wgrad is in wgrad.hip).

extern "C" int moe_grouped_fc2_dgrad_dswiglu(const void* dy, const uint8_t* dy_scales, int fmt,
                                             const void* w2t, const uint8_t* w2t_scales,
                                             const int32_t* offsets, int E, int H, int F,
                                             int64_t rows, const float* act_save, void* da,
                                             uint8_t* da_scales, float* da_f32,
                                             hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(E >= 1 && E <= kMaxGroups && H > 0 && F > 0 && rows >= 0, MOE_ERR_INVALID_ARG,
              "moe_grouped_fc2_dgrad_dswiglu: need 1 <= E <= 1024, H > 0, F > 0, rows >= 0");
  MOE_REQUIRE(fmt == MOE_BF16 || fmt == MOE_MXFP8_E4M3 || fmt == MOE_MXFP4_E2M1, MOE_ERR_UNSUPPORTED,
              "moe_grouped_fc2_dgrad_dswiglu: fmt must be BF16, MXFP8 or MXFP4");
  const int kmul = fmt == MOE_MXFP4_E2M1 ? 256 : 128;
  MOE_REQUIRE(H % kmul == 0 && F % 128 == 0, MOE_ERR_INVALID_ARG,
              "moe_grouped_fc2_dgrad_dswiglu: need H % 128 == 0 (256 for MXFP4) and F % 128 == 0");
  MOE_REQUIRE(offsets && w2t && act_save && da && (rows == 0 || dy), MOE_ERR_INVALID_ARG,
              "moe_grouped_fc2_dgrad_dswiglu: null pointer");
  if (is_mx(fmt))
    MOE_REQUIRE(dy_scales && w2t_scales && da_scales && scale_aligned(dy_scales) &&
                    scale_aligned(w2t_scales),
                MOE_ERR_INVALID_ARG, "moe_grouped_fc2_dgrad_dswiglu: MX needs 4-byte aligned scales");
  MOE_REQUIRE(aligned16(dy) && aligned16(w2t) && aligned16(act_save) && aligned16(da) &&
                  (!da_f32 || aligned16(da_f32)),
              MOE_ERR_ALIGNMENT, "moe_grouped_fc2_dgrad_dswiglu: tensors must be 16-byte aligned");
  if (rows == 0) return MOE_OK;
  return expert_gemm(2, dy, dy_scales, fmt, nullptr, w2t, w2t_scales, offsets, E, F, H, rows, F,
                     da, da_scales, nullptr, act_save, da_f32, stream);
}

extern "C" int moe_grouped_fc1_dgrad(const void* da, const uint8_t* da_scales, int fmt,
                                     const void* w1t, const uint8_t* w1t_scales,
                                     const int32_t* offsets, int E, int H, int F, int64_t rows,
                                     void* dx_perm, hipStream_t stream) {
  // dX rows = dA . W1 with W1 stored transposed [E, H, 2F] (contraction over
  // 2F contiguous): the fc2 kernel with 2F in place of F.
  clear_error();
  MOE_REQUIRE(E >= 1 && E <= kMaxGroups && H > 0 && F > 0 && rows >= 0, MOE_ERR_INVALID_ARG,
              "moe_grouped_fc1_dgrad: need 1 <= E <= 1024, H > 0, F > 0, rows >= 0");
  MOE_REQUIRE(fmt == MOE_BF16 || fmt == MOE_MXFP8_E4M3 || fmt == MOE_MXFP4_E2M1, MOE_ERR_UNSUPPORTED,
              "moe_grouped_fc1_dgrad: fmt must be BF16, MXFP8 or MXFP4");
  int st = check_formats("moe_grouped_fc1_dgrad", fmt, fmt, MOE_BF16, H, 2 * F);
  if (st) return st;
  MOE_REQUIRE(offsets && w1t && dx_perm && (rows == 0 || da), MOE_ERR_INVALID_ARG,
              "moe_grouped_fc1_dgrad: null pointer");
  if (is_mx(fmt))
    MOE_REQUIRE(da_scales && w1t_scales && scale_aligned(da_scales) && scale_aligned(w1t_scales),
                MOE_ERR_INVALID_ARG, "moe_grouped_fc1_dgrad: MX needs 4-byte aligned scales");
  MOE_REQUIRE(aligned16(da) && aligned16(w1t) && aligned16(dx_perm), MOE_ERR_ALIGNMENT,
              "moe_grouped_fc1_dgrad: tensors must be 16-byte aligned");
  if (rows == 0) return MOE_OK;
  return fc2_impl(da, da_scales, fmt, w1t, w1t_scales, offsets, E, H, 2 * F, rows, dx_perm, stream);
}

// ---------------------------------------------------------------------------
// NVFP4 W4A4 grouped MLP (page "Mistral Large 3 NVFP4 TRTLLM MoE support",
// title and Modifications): E2M1 weights with E4M3 scales per 16 and one fp32
// scale per expert matrix, streamed 4-bit and converted to exact bf16 values
// in registers for bf16 matrix instructions; activations as bf16 operand
// values code * scale; every tensor scale applied to the fp32 accumulators.

static int check_nvfp4(const char* fn, int E, int H, int F, int64_t rows) {
  std::string f(fn);
  MOE_REQUIRE(E >= 1 && E <= kMaxGroups && H > 0 && F > 0 && rows >= 0, MOE_ERR_INVALID_ARG,
              f + ": need 1 <= E <= 1024, H > 0, F > 0, rows >= 0");
  MOE_REQUIRE(H % 128 == 0 && F % 64 == 0, MOE_ERR_INVALID_ARG,
              f + ": NVFP4 needs H % 128 == 0 and F % 64 == 0");
  return MOE_OK;
}

extern "C" int moe_grouped_fc1_swiglu_nvfp4(const void* a_vals, const int32_t* src_row,
                                            const void* w1, const uint8_t* w1_scales,
                                            const float* w1_g, float x_g, float h_g,
                                            const int32_t* offsets, int E, int H, int F,
                                            int64_t rows, void* h_vals, hipStream_t stream) {
  clear_error();
  int st = check_nvfp4("moe_grouped_fc1_swiglu_nvfp4", E, H, F, rows);
  if (st) return st;
  if (rows == 0) return MOE_OK;
  MOE_REQUIRE(a_vals && w1 && w1_scales && w1_g && offsets && h_vals, MOE_ERR_INVALID_ARG,
              "moe_grouped_fc1_swiglu_nvfp4: null pointer");
  MOE_REQUIRE(aligned16(a_vals) && aligned16(w1) && aligned16(h_vals) && scale_aligned(w1_scales),
              MOE_ERR_ALIGNMENT,
              "moe_grouped_fc1_swiglu_nvfp4: tensors 16-byte, weight scales 4-byte aligned");
  MOE_REQUIRE(x_g > 0.f && h_g > 0.f, MOE_ERR_INVALID_ARG,
              "moe_grouped_fc1_swiglu_nvfp4: tensor scales must be positive");
  const NvScales nv{x_g, w1_g, h_g};
  return expert_gemm(0, a_vals, nullptr, MOE_NVFP4_E2M1, src_row, w1, w1_scales, offsets, E, 2 * F, H,
                     rows, F, h_vals, nullptr, nullptr, nullptr, nullptr, stream, nullptr, &nv);
}

extern "C" int moe_grouped_fc2_nvfp4(const void* h_vals, const void* w2, const uint8_t* w2_scales,
                                     const float* w2_g, float h_g, const int32_t* offsets, int E,
                                     int H, int F, int64_t rows, void* y, hipStream_t stream) {
  clear_error();
  int st = check_nvfp4("moe_grouped_fc2_nvfp4", E, H, F, rows);
  if (st) return st;
  if (rows == 0) return MOE_OK;
  MOE_REQUIRE(h_vals && w2 && w2_scales && w2_g && offsets && y, MOE_ERR_INVALID_ARG,
              "moe_grouped_fc2_nvfp4: null pointer");
  MOE_REQUIRE(aligned16(h_vals) && aligned16(w2) && aligned16(y) && scale_aligned(w2_scales),
              MOE_ERR_ALIGNMENT, "moe_grouped_fc2_nvfp4: tensors 16-byte, weight scales 4-byte aligned");
  MOE_REQUIRE(h_g > 0.f, MOE_ERR_INVALID_ARG, "moe_grouped_fc2_nvfp4: tensor scale must be positive");
  const NvScales nv{h_g, w2_g, 0.f};
  return expert_gemm(1, h_vals, nullptr, MOE_NVFP4_E2M1, nullptr, w2, w2_scales, offsets, E, H, F,
                     rows, 0, y, nullptr, nullptr, nullptr, nullptr, stream, nullptr, &nv);
}
