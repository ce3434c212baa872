// Launcher of the grouped expert GEMM (expert_gemm.hip), shared by the entry
// points of grouped_mlp.hip.
#pragma once

#include "common.h"

namespace moe {

// An always-on expert (the layer's shared expert) run by the same launch as
// the routed experts: `rows` rows whose A operand rows start at `a_row0` and
// whose output rows start at `row0`, packed weights `w` (+ MX `w_scales`)
// in the routed experts' format and shape.
struct DenseExpert {
  const void* w;
  const uint8_t* w_scales;
  int rows;
  int row0;
  int a_row0;
};

// Tensor scales of the NVFP4 layer: of the activation operand, of each
// expert's weight matrix (device array [E]) and of the fc1 output h.
struct NvScales {
  float a_g;
  const float* w_g;
  float out_g;
};

// kind: 0 fc1 + SwiGLU (N = 2F, out = h), 1 plain (out = y bf16), 2 dSwiGLU
// (N = F, out = dA). Arguments are validated by the callers. NVFP4 (fmt
// MOE_NVFP4_E2M1): the activation operand is bf16 values code * scale, the
// weights packed E2M1 + E4M3 (moe_pack_weights), kinds 0 and 1 only, no
// dense expert, `nv` required; fc1's h is written as bf16 operand values.
int expert_gemm(int kind, const void* a, const uint8_t* a_scales, int fmt, const int32_t* gather,
                const void* wp, const uint8_t* wp_scales, const int32_t* offsets, int E, int N,
                int K, int64_t rows, int half, void* out, uint8_t* out_scales, float* act_save,
                const float* a_saved, float* da_f32, hipStream_t stream,
                const DenseExpert* dense = nullptr, const NvScales* nv = nullptr);

}  // namespace moe
