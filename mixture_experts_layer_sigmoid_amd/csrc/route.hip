// moe_route: router GEMM + sigmoid + selection bias + grouped top-k +
// normalized, scaled combine weights, fused in one kernel.
//
// Method: page "[PyTorch] DeepSeekV3Layer: full MoE transformer layer (MLA +
// DeepSeek MoE)", Description, DeepSeekV3MoE item ("fused sigmoid router
// with aux-loss-free bias and grouped top-k"). Readings where that page is
// silent: group score = sum of the two largest biased scores of the group;
// dropped groups are excluded (-inf); ties go to the lower group / expert
// index; outputs are in descending order of the biased score; the weights
// use the unbiased scores, normalized then scaled; the sigmoid is evaluated
// in fp64 and rounded once to fp32.
//
// Layout of the work: one workgroup of 4 wavefronts handles 16 tokens. The
// logits tile [16, E] is produced by MFMA (bf16 16x16x32, tokens in M,
// experts in N, each wave owning every 4th 16-expert block) or by fp32 FMA,
// and kept in LDS. Selection then runs one wavefront per token with the E
// scores spread over the 64 lanes (expert e on lane e % 64); every argmax is
// a 64-lane max-reduction of a 64-bit key (order-preserving score bits in
// the high word, the complemented index in the low word, which turns "ties
// to the lower index" into a plain max).
#include "common.h"

#include <cmath>

namespace moe {
namespace {

constexpr int kTokPerBlock = 16;
constexpr int kThreads = 256;
constexpr int kMaxE = 512;
constexpr int kMaxPerLane = kMaxE / 64;

__device__ __forceinline__ uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    unsigned long long o = __shfl_xor(v, m, 64);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ unsigned long long make_key(float score, int index) {
  return (static_cast<unsigned long long>(orderable(score)) << 32) |
         static_cast<unsigned long long>(~static_cast<uint32_t>(index));
}

__device__ __forceinline__ int key_index(unsigned long long key) {
  return static_cast<int>(~static_cast<uint32_t>(key & 0xFFFFFFFFull));
}

// Logits of 16 tokens x E experts, bf16 inputs, fp32 MFMA accumulation.
__device__ void logits_bf16(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                            int T, int H, int E, int t0, float* lg /* LDS [16][E] */) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nblk = (E + 15) / 16;
  const int row = lane & 15;
  const int kq = (lane >> 4) * 8;  // k offset of this lane inside a 32-wide step
  const int tok = min(t0 + row, T - 1);
  const uint16_t* xa = x + static_cast<int64_t>(tok) * H + kq;
  constexpr int kMaxBlkPerWave = kMaxE / 16 / 4;
  f32x4_t acc[kMaxBlkPerWave];
  const uint16_t* wb[kMaxBlkPerWave];
  int myblk = 0;
#pragma unroll
  for (int i = 0; i < kMaxBlkPerWave; ++i) {
    acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    int nb = wave + 4 * i;
    int ex = min(nb * 16 + row, E - 1);
    wb[i] = wr + static_cast<int64_t>(ex) * H + kq;
    if (nb < nblk) myblk = i + 1;
  }
  for (int k0 = 0; k0 < H; k0 += 32) {
    bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(xa + k0);
#pragma unroll
    for (int i = 0; i < kMaxBlkPerWave; ++i) {
      if (i < myblk) {
        bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(wb[i] + k0);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
      }
    }
  }
  // C layout of 16x16 MFMA: lane l, element r -> row 4*(l/16)+r, column l%16
#pragma unroll
  for (int i = 0; i < kMaxBlkPerWave; ++i) {
    if (i < myblk) {
      int col = (wave + 4 * i) * 16 + (lane & 15);
      if (col < E) {
#pragma unroll
        for (int r = 0; r < 4; ++r) lg[(4 * (lane >> 4) + r) * E + col] = acc[i][r];
      }
    }
  }
}

// Logits with fp32 inputs by plain FMA (the small fp32 layer).
__device__ void logits_f32(const float* __restrict__ x, const float* __restrict__ wr, int T,
                           int H, int E, int t0, float* lg) {
  for (int o = threadIdx.x; o < kTokPerBlock * E; o += kThreads) {
    int r = o / E, e = o % E;
    int tok = min(t0 + r, T - 1);
    const float* xp = x + static_cast<int64_t>(tok) * H;
    const float* wp = wr + static_cast<int64_t>(e) * H;
    float acc = 0.f;
    for (int h = 0; h < H; ++h) acc = fmaf(xp[h], wp[h], acc);
    lg[r * E + e] = acc;
  }
}

template <int XFMT>
__global__ __launch_bounds__(kThreads) void route_kernel(
    const void* __restrict__ x, const void* __restrict__ wr, const float* __restrict__ bias,
    const float* __restrict__ logits_in, int T, int H, int E, int n_group, int topk_group,
    int k, float routed_scale, float* __restrict__ logits_out, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w) {
  __shared__ float lg[kTokPerBlock * kMaxE];
  __shared__ float s_sc[4][kMaxE];   // per wave: sigmoid scores of its token
  __shared__ float s_sel[4][kMaxE];  // per wave: biased scores of its token
  const int t0 = blockIdx.x * kTokPerBlock;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  if (logits_in == nullptr) {
    if (XFMT == MOE_BF16)
      logits_bf16(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wr), T, H, E, t0, lg);
    else
      logits_f32(static_cast<const float*>(x), static_cast<const float*>(wr), T, H, E, t0, lg);
    __syncthreads();
  }

  const int G = E / n_group;
  for (int r = wave; r < kTokPerBlock; r += 4) {
    const int t = t0 + r;
    if (t >= T) break;
    // scores of this token, expert e on lane e % 64
    float val[kMaxPerLane];
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      int e = lane + 64 * i;
      val[i] = -INFINITY;
      if (e < E) {
        float l = logits_in ? logits_in[static_cast<int64_t>(t) * E + e] : lg[r * E + e];
        if (logits_out) logits_out[static_cast<int64_t>(t) * E + e] = l;
        float s = static_cast<float>(1.0 / (1.0 + exp(-static_cast<double>(l))));
        float sel = s + bias[e];
        s_sc[wave][e] = s;
        s_sel[wave][e] = sel;
        val[i] = sel;
      }
    }
    if (n_group > 1) {
      __builtin_amdgcn_wave_barrier();
      // group q on lane q: the two largest biased scores of the group
      float gscore = -INFINITY;
      if (lane < n_group) {
        float m1 = -INFINITY, m2 = -INFINITY;
        for (int e = lane * G; e < (lane + 1) * G; ++e) {
          float v = s_sel[wave][e];
          if (v > m1) {
            m2 = m1;
            m1 = v;
          } else if (v > m2) {
            m2 = v;
          }
        }
        gscore = m1 + m2;
      }
      unsigned long long kept = 0;  // bit q set: group q kept
      for (int i = 0; i < topk_group; ++i) {
        unsigned long long key = lane < n_group ? make_key(gscore, lane) : 0ull;
        int q = key_index(wave_max_u64(key));
        kept |= 1ull << q;
        if (lane == q) gscore = -INFINITY;
      }
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i) {
        int e = lane + 64 * i;
        if (e < E && !((kept >> (e / G)) & 1ull)) val[i] = -INFINITY;
      }
    }
    // top-k by repeated 64-lane argmax
    int my_idx = 0;
    for (int j = 0; j < k; ++j) {
      unsigned long long best = 0;
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i) {
        int e = lane + 64 * i;
        if (e < E) {
          unsigned long long key = make_key(val[i], e);
          best = key > best ? key : best;
        }
      }
      int e = key_index(wave_max_u64(best));
      if (lane == j) my_idx = e;
      if (lane == (e & 63)) {
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i)
          if (i == (e >> 6)) val[i] = -INFINITY;
      }
    }
    // normalize the unbiased scores of the chosen experts, then scale
    float S = 0.f;
    for (int j = 0; j < k; ++j) {
      int e = __shfl(my_idx, j, 64);
      S += s_sc[wave][e];
    }
    if (lane < k) {
      float w = s_sc[wave][my_idx] / S;
      topk_idx[static_cast<int64_t>(t) * k + lane] = my_idx;
      topk_w[static_cast<int64_t>(t) * k + lane] = w * routed_scale;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_route(const void* x, int x_fmt, const void* w_router, const float* bias,
                         const float* logits_in, int T, int H, int E, int n_group,
                         int topk_group, int k, float routed_scale, float* logits_out,
                         int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(T >= 0, MOE_ERR_INVALID_ARG, "moe_route: T < 0");
  MOE_REQUIRE(E >= 1 && E <= kMaxE, MOE_ERR_INVALID_ARG, "moe_route: E must be in [1, 512]");
  MOE_REQUIRE(n_group >= 1 && n_group <= 64 && E % n_group == 0, MOE_ERR_INVALID_ARG,
              "moe_route: n_group must divide E and be <= 64");
  MOE_REQUIRE(n_group == 1 || E / n_group >= 2, MOE_ERR_INVALID_ARG,
              "moe_route: groups need at least 2 experts");
  MOE_REQUIRE(topk_group >= 1 && topk_group <= n_group, MOE_ERR_INVALID_ARG,
              "moe_route: topk_group must be in [1, n_group]");
  MOE_REQUIRE(k >= 1 && k <= 16 && k <= topk_group * (E / n_group), MOE_ERR_INVALID_ARG,
              "moe_route: k must be in [1, min(16, topk_group * E / n_group)]");
  MOE_REQUIRE(bias && topk_idx && topk_w, MOE_ERR_INVALID_ARG,
              "moe_route: bias, topk_idx and topk_w are required");
  if (!logits_in) {
    MOE_REQUIRE(x && w_router, MOE_ERR_INVALID_ARG,
                "moe_route: x and w_router are required without logits_in");
    MOE_REQUIRE(x_fmt == MOE_F32 || x_fmt == MOE_BF16, MOE_ERR_UNSUPPORTED,
                "moe_route: x_fmt must be MOE_F32 or MOE_BF16");
    MOE_REQUIRE(H >= 1, MOE_ERR_INVALID_ARG, "moe_route: H < 1");
    if (x_fmt == MOE_BF16) {
      MOE_REQUIRE(H % 32 == 0, MOE_ERR_INVALID_ARG, "moe_route: bf16 needs H % 32 == 0");
      MOE_REQUIRE(aligned16(x) && aligned16(w_router), MOE_ERR_ALIGNMENT,
                  "moe_route: x and w_router must be 16-byte aligned");
    }
  }
  if (T == 0) return MOE_OK;
  dim3 grid((T + kTokPerBlock - 1) / kTokPerBlock), block(kThreads);
  if (logits_in || x_fmt == MOE_F32)
    hipLaunchKernelGGL(route_kernel<MOE_F32>, grid, block, 0, stream, x, w_router, bias, logits_in,
                       T, H, E, n_group, topk_group, k, routed_scale, logits_out, topk_idx, topk_w);
  else
    hipLaunchKernelGGL(route_kernel<MOE_BF16>, grid, block, 0, stream, x, w_router, bias,
                       logits_in, T, H, E, n_group, topk_group, k, routed_scale, logits_out,
                       topk_idx, topk_w);
  return check_launch("moe_route");
}
