// moe_grouped_mlp_bwd: the whole backward of the routed expert path as one
// call on caller-provided scratch.
//
// Page "[PyTorch] DeepSeekV3Layer: full MoE transformer layer (MLA +
// DeepSeek MoE)", Performance section, "Where the time goes": the fused
// grouped MLP's dGLU backward and wgrad in MXFP8, and the local permute's
// reduce (the un-permute of dX). Routing weights are constants and the
// quantizers pass gradients straight through.
//
// The call enqueues, on one stream:
//   combine backward (dY rows = w * dOut, MX-encoded from the fp32 products,
//     plus each row's weight)
//   -> fc2 data gradient fused with the SwiGLU backward (dA in MX + fp32)
//   -> fc1 data gradient (dX rows, bf16) -> summing un-permute (dX, bf16)
//   -> stage-major MX operands of the weight gradients (dY from dOut and the
//      row weights, h recomputed from the saved fc1 output, dA from its fp32
//      copy, x) -> dW2 = dY^T h and dW1 = dA^T x per expert.
// Every argument is checked on the host before the first kernel is
// enqueued. The scratch holds what lives across phases (segment starts, row
// weights, the fp32 dA) and, in one region reused by both phases, the
// data-gradient buffers and then the weight-gradient operands.
#include "common.h"

#include <algorithm>
#include <string>

namespace moe {
namespace {

constexpr int kMaxE = 1024;

size_t up256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

// byte offsets of the scratch buffers
struct BwdLayout {
  int64_t kstride;
  size_t kofs, row_w, da_f32;                                   // persistent
  size_t dy_q, dy_sc, da, da_sc, dx_perm;                       // data-gradient phase
  size_t dyT, dyT_sc, hT, hT_sc, daT, daT_sc, xT, xT_sc;        // weight-gradient phase
  size_t total;
};

BwdLayout bwd_layout(int E, int H, int F, int64_t rows) {
  BwdLayout L{};
  const size_t R = static_cast<size_t>(rows);
  L.kstride = moe_segments_kstride(rows, E);
  const size_t ks = static_cast<size_t>(L.kstride);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += up256(bytes);
    return at;
  };
  L.kofs = take((E + 1) * sizeof(int32_t));
  L.row_w = take(R * sizeof(float));
  L.da_f32 = take(R * 2 * F * sizeof(float));
  const size_t shared = o;
  L.dy_q = take(R * H);
  L.dy_sc = take(R * (H / 32));
  L.da = take(R * 2 * F);
  L.da_sc = take(R * (2 * F / 32));
  L.dx_perm = take(R * H * 2);
  const size_t end_a = o;
  o = shared;
  L.dyT = take(static_cast<size_t>(H) * ks);
  L.dyT_sc = take(static_cast<size_t>(H) * (ks / 32));
  L.hT = take(static_cast<size_t>(F) * ks);
  L.hT_sc = take(static_cast<size_t>(F) * (ks / 32));
  L.daT = take(static_cast<size_t>(2 * F) * ks);
  L.daT_sc = take(static_cast<size_t>(2 * F) * (ks / 32));
  L.xT = take(static_cast<size_t>(H) * ks);
  L.xT_sc = take(static_cast<size_t>(H) * (ks / 32));
  L.total = std::max(end_a, o);
  return L;
}

bool shapes_ok(int T, int k, int E, int H, int F, int64_t rows) {
  return T >= 0 && k >= 1 && k <= 16 && E >= 1 && E <= kMaxE && H > 0 && F > 0 &&
         H % 128 == 0 && F % 128 == 0 && rows >= static_cast<int64_t>(T) * k &&
         rows < (int64_t{1} << 31);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_grouped_mlp_bwd_workspace(int T, int k, int E, int H, int F, int64_t rows,
                                                int fmt) {
  if (fmt != MOE_MXFP8_E4M3 || !shapes_ok(T, k, E, H, F, rows)) return 0;
  return bwd_layout(E, H, F, rows).total;
}

extern "C" int moe_grouped_mlp_bwd(const void* dout, const void* x, int act_fmt,
                                   const int32_t* row_map, const int32_t* src_row,
                                   const float* topk_w, const int32_t* offsets,
                                   const float* act_save, const void* w1t,
                                   const uint8_t* w1t_scales, const void* w2t,
                                   const uint8_t* w2t_scales, int fmt, int T, int k, int E, int H,
                                   int F, int64_t rows, void* dx, void* dw1, void* dw2, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(shapes_ok(T, k, E, H, F, rows), MOE_ERR_INVALID_ARG,
              "moe_grouped_mlp_bwd: need T >= 0, 1 <= k <= 16, 1 <= E <= 1024, H and F positive "
              "multiples of 128, T * k <= rows < 2^31");
  MOE_REQUIRE(fmt == MOE_MXFP8_E4M3, MOE_ERR_UNSUPPORTED,
              "moe_grouped_mlp_bwd: the backward runs in MXFP8 (fmt MOE_MXFP8_E4M3)");
  MOE_REQUIRE(act_fmt == MOE_BF16 || act_fmt == MOE_F32, MOE_ERR_UNSUPPORTED,
              "moe_grouped_mlp_bwd: act_fmt (dout, x, dx) must be MOE_BF16 or MOE_F32");
  MOE_REQUIRE(src_row && offsets && act_save && w1t && w1t_scales && w2t && w2t_scales && dw1 &&
                  dw2 && (T == 0 || (dout && x && row_map && topk_w && dx)),
              MOE_ERR_INVALID_ARG, "moe_grouped_mlp_bwd: null pointer");
  MOE_REQUIRE(aligned16(act_save) && aligned16(w1t) && aligned16(w2t) && aligned16(dw1) &&
                  aligned16(dw2) && (T == 0 || (aligned16(dout) && aligned16(x) && aligned16(dx))),
              MOE_ERR_ALIGNMENT, "moe_grouped_mlp_bwd: tensors must be 16-byte aligned");
  MOE_REQUIRE((reinterpret_cast<uintptr_t>(w1t_scales) & 3u) == 0 &&
                  (reinterpret_cast<uintptr_t>(w2t_scales) & 3u) == 0,
              MOE_ERR_ALIGNMENT, "moe_grouped_mlp_bwd: weight scales must be 4-byte aligned");
  const BwdLayout L = bwd_layout(E, H, F, rows);
  MOE_REQUIRE(ws && ws_bytes >= L.total && aligned16(ws), MOE_ERR_WORKSPACE,
              "moe_grouped_mlp_bwd: workspace missing, unaligned or smaller than "
              "moe_grouped_mlp_bwd_workspace(T, k, E, H, F, rows, fmt) = " +
                  std::to_string(L.total) + " bytes");

  uint8_t* w = static_cast<uint8_t*>(ws);
  auto at = [&](size_t off) { return w + off; };
  int32_t* kofs = reinterpret_cast<int32_t*>(at(L.kofs));
  float* row_w = reinterpret_cast<float*>(at(L.row_w));
  float* da_f32 = reinterpret_cast<float*>(at(L.da_f32));
  // with no tokens there is nothing to read; any valid address stands in
  const void* dout_p = T > 0 ? dout : ws;
  const void* x_p = T > 0 ? x : ws;
  const int f8 = MOE_MXFP8_E4M3;
  const int64_t ks = L.kstride;
  int st;
  // data gradients
  st = moe_combine_bwd(dout_p, act_fmt, row_map, src_row, topk_w, T, k, H, rows, at(L.dy_q), f8,
                       at(L.dy_sc), row_w, stream);
  if (st) return st;
  st = moe_grouped_fc2_dgrad_dswiglu(at(L.dy_q), at(L.dy_sc), f8, w2t, w2t_scales, offsets, E, H,
                                     F, rows, act_save, at(L.da), at(L.da_sc), da_f32, stream);
  if (st) return st;
  st = moe_grouped_fc1_dgrad(at(L.da), at(L.da_sc), f8, w1t, w1t_scales, offsets, E, H, F, rows,
                             at(L.dx_perm), stream);
  if (st) return st;
  st = moe_unpermute(at(L.dx_perm), MOE_BF16, row_map, T, k, H, dx, act_fmt, stream);
  if (st) return st;
  // weight gradients (their operands overwrite the data-gradient buffers)
  st = moe_quantize_mx_segments(dout_p, act_fmt, 1, src_row, offsets, row_w, E, rows, H, ks, f8,
                                at(L.dyT), at(L.dyT_sc), kofs, stream);
  if (st) return st;
  st = moe_quantize_mx_segments(act_save, MOE_F32, 2, src_row, offsets, nullptr, E, rows, F, ks,
                                f8, at(L.hT), at(L.hT_sc), kofs, stream);
  if (st) return st;
  st = moe_grouped_wgrad(at(L.dyT), at(L.dyT_sc), at(L.hT), at(L.hT_sc), f8, kofs, E, H, F, ks,
                         dw2, stream);
  if (st) return st;
  st = moe_quantize_mx_segments(da_f32, MOE_F32, 0, src_row, offsets, nullptr, E, rows, 2 * F, ks,
                                f8, at(L.daT), at(L.daT_sc), kofs, stream);
  if (st) return st;
  st = moe_quantize_mx_segments(x_p, act_fmt, 1, src_row, offsets, nullptr, E, rows, H, ks, f8,
                                at(L.xT), at(L.xT_sc), kofs, stream);
  if (st) return st;
  return moe_grouped_wgrad(at(L.daT), at(L.daT_sc), at(L.xT), at(L.xT_sc), f8, kofs, E, 2 * F, H,
                           ks, dw1, stream);
}
