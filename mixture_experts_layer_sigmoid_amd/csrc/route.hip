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
// Layout of the work, two kernels:
//  * router GEMM: logits = x . W_r^T, split along H into S chunks so the
//    launch has a few hundred workgroups whatever T; partial sums go to a
//    workspace [S, T, E] fp32. bf16 with H % 64 == 0: tiles of 64 tokens x
//    256 experts, both operands staged through two LDS buffers of 64 K
//    values (direct global->LDS loads, XOR-swizzled rows), each wave owning
//    64 tokens x 64 experts as 2 x 2 blocks of 32x32x16 bf16 MFMAs; other
//    bf16 shapes: MFMA 16x16x32 straight from global memory; fp32: plain
//    FMA.
//  * selection: one wavefront per token sums the S partials in chunk order
//    and spreads the E scores over the 64 lanes (expert e on lane e % 64);
//    every argmax is a 64-lane max-reduction of a 64-bit key
//    (order-preserving score bits in the high word, the complemented index
//    in the low word, which turns "ties to the lower index" into a plain
//    max).
#include "common.h"
#include "gemm_util.h"

#include <algorithm>
#include <cmath>

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxE = 512;
constexpr int kMaxPerLane = kMaxE / 64;
constexpr int kTile = 64;       // tokens and experts per router GEMM tile
constexpr int kMinChunk = 128;  // smallest H chunk of the split
constexpr int kTargetWgs = 512;

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

// Partial logits of one tile over H chunk [k0, k1):
// part[s, t, e] = sum_{h in chunk} x[t, h] * w[e, h].
template <int XFMT>
__global__ __launch_bounds__(kThreads) void router_gemm_kernel(const void* __restrict__ x,
                                                               const void* __restrict__ wr, int T,
                                                               int H, int E, int chunk, int S,
                                                               float* __restrict__ part) {
  const int ne = (E + kTile - 1) / kTile;
  int b = blockIdx.x;
  const int s = b % S;
  b /= S;
  const int t0 = (b / ne) * kTile, e0 = (b % ne) * kTile;
  const int k0 = s * chunk, k1 = min(H, k0 + chunk);
  float* out = part + static_cast<int64_t>(s) * T * E;
  if constexpr (XFMT == MOE_BF16) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kq = (lane >> 4) * 8;  // k offset of this lane inside a 32-wide step
    const int tok = min(t0 + 16 * wave + (lane & 15), T - 1);
    const uint16_t* xa = static_cast<const uint16_t*>(x) + static_cast<int64_t>(tok) * H + kq;
    const uint16_t* wb[4];
    f32x4_t acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ex = min(e0 + 16 * j + (lane & 15), E - 1);
      wb[j] = static_cast<const uint16_t*>(wr) + static_cast<int64_t>(ex) * H + kq;
      acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll 4
    for (int k = k0; k < k1; k += 32) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(xa + k);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8_t w = *reinterpret_cast<const bf16x8_t*>(wb[j] + k);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, w, acc[j], 0, 0, 0);
      }
    }
    // C layout of 16x16 MFMA: lane l, element r -> row 4*(l/16)+r, column l%16
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + 16 * j + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 16 * wave + 4 * (lane >> 4) + r;
        if (t < T && e < E) out[static_cast<int64_t>(t) * E + e] = acc[j][r];
      }
    }
  } else {
    const float* xf = static_cast<const float*>(x);
    const float* wf = static_cast<const float*>(wr);
    for (int o = threadIdx.x; o < kTile * kTile; o += kThreads) {
      const int t = t0 + o / kTile, e = e0 + o % kTile;
      if (t >= T || e >= E) continue;
      const float* xp = xf + static_cast<int64_t>(t) * H;
      const float* wp = wf + static_cast<int64_t>(e) * H;
      float acc = 0.f;
      for (int h = k0; h < k1; ++h) acc = fmaf(xp[h], wp[h], acc);
      out[static_cast<int64_t>(t) * E + e] = acc;
    }
  }
}

// Partial logits over H chunk [k0, k1) (a multiple of 64) for a tile of 64
// tokens x 256 experts: part[s, t, e] = sum_{h in chunk} x[t, h] * w[e, h].
// Rows past T or E load the last valid row and are not stored.
constexpr int kRtTok = 64, kRtExp = 256, kRtK = 64;   // tile and stage (bf16 values)
constexpr int kRtRowB = kRtK * 2;                     // bytes per row per stage
constexpr int kRtStage = (kRtTok + kRtExp) * kRtRowB;  // 40 KB
__global__ __launch_bounds__(kThreads) void router_mfma_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ wr,
                                                               int T, int H, int E, int chunk,
                                                               int S, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kRtStage];
  const int ne = (E + kRtExp - 1) / kRtExp;
  int b = blockIdx.x;
  const int s = b % S;
  b /= S;
  const int t0 = (b / ne) * kRtTok, e0 = (b % ne) * kRtExp;
  const int k0 = s * chunk, k1 = min(H, k0 + chunk);
  const int KT = (k1 - k0) / kRtK;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  // loads: instruction q covers 8 rows x 128 bytes; rows 0..63 are tokens
  // (q = 0..7), 64..319 experts (q = 8..39); wave w issues q = w + 4i
  const uint16_t* src[10];
  int dst[10];
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const int q = wave + 4 * i;
    const int r = 8 * q + (lane >> 3);
    const int chunk16 = (lane & 7) ^ swz_key<128>(r);
    const uint16_t* row = r < kRtTok ? x + static_cast<int64_t>(min(t0 + r, T - 1)) * H
                                     : wr + static_cast<int64_t>(min(e0 + r - kRtTok, E - 1)) * H;
    src[i] = row + k0 + chunk16 * 8;
    dst[i] = q * 1024;
  }
  auto issue = [&](int kt) {
    uint8_t* st = smem + (kt & 1) * kRtStage;
#pragma unroll
    for (int i = 0; i < 10; ++i) lds_load16(src[i] + kt * kRtK, st + dst[i]);
  };
  f32x16_t acc[2][2];  // [token block][expert block]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};
  issue(0);
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) {
      issue(kt + 1);
      wait_vmcnt<10>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    const uint8_t* st = smem + (kt & 1) * kRtStage;
#pragma unroll
    for (int ks = 0; ks < kRtK / 16; ++ks) {
      bf16x8_t a[2], w[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = *reinterpret_cast<const bf16x8_t*>(st + swz<128>(32 * i + (lane & 31), 2 * ks + g));
        const int er = kRtTok + 64 * wave + 32 * i + (lane & 31);
        w[i] = *reinterpret_cast<const bf16x8_t*>(st + swz<128>(er, 2 * ks + g));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[j], a[i], acc[i][j], 0, 0, 0);
    }
    lds_barrier();  // the buffer is reloaded by the next iteration's issue
  }
  // accumulator of block (i, j): lane l holds token 32 i + l % 32 and, in
  // element r, expert 64 wave + 32 j + 8 (r / 4) + 4 (l / 32) + r % 4
  float* out = part + static_cast<int64_t>(s) * T * E;
  const int t = t0 + (lane & 31);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (t + 32 * i >= T) continue;
    float* orow = out + static_cast<int64_t>(t + 32 * i) * E;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = e0 + 64 * wave + 32 * j + 8 * q + 4 * g;
        if (e + 3 < E && (E & 3) == 0) {
          *reinterpret_cast<f32x4_t*>(orow + e) =
              f32x4_t{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (e + r < E) orow[e + r] = acc[i][j][4 * q + r];
        }
      }
  }
}

// One wavefront per token: logits (sum of S partials, or logits_in), then
// sigmoid, bias, group limit, top-k and the combine weights.
__global__ __launch_bounds__(kThreads) void select_kernel(
    const float* __restrict__ part, int S, const float* __restrict__ bias, int T, int E,
    int n_group, int topk_group, int k, float routed_scale, float* __restrict__ logits_out,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  __shared__ float s_sc[4][kMaxE];   // per wave: sigmoid scores of its token
  __shared__ float s_sel[4][kMaxE];  // per wave: biased scores of its token
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;  // no block-level barrier below
  // scores of this token, expert e on lane e % 64
  float val[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    val[i] = -INFINITY;
    if (e < E) {
      const float* pe = part + static_cast<int64_t>(t) * E + e;
      const int64_t ps = static_cast<int64_t>(T) * E;   // between partials
      float l;
      if (S == 1) {
        l = pe[0];
      } else {
        // eight independent running sums, so eight partials per step are in
        // flight instead of one dependent load at a time (a decode batch
        // splits H over dozens of partials)
        float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        int s = 0;
        for (; s + 8 <= S; s += 8) {
#pragma unroll
          for (int u = 0; u < 8; ++u) a[u] += pe[(s + u) * ps];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (s + u < S) a[u] += pe[(s + u) * ps];
        l = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
      }
      if (logits_out) logits_out[static_cast<int64_t>(t) * E + e] = l;
      const float sc = static_cast<float>(1.0 / (1.0 + exp(-static_cast<double>(l))));
      const float sel = sc + bias[e];
      s_sc[wave][e] = sc;
      s_sel[wave][e] = sel;
      val[i] = sel;
    }
  }
  __builtin_amdgcn_wave_barrier();
  if (n_group > 1) {
    const int G = E / n_group;
    // group q on lane q: the two largest biased scores of the group
    float gscore = -INFINITY;
    if (lane < n_group) {
      float m1 = -INFINITY, m2 = -INFINITY;
      for (int e = lane * G; e < (lane + 1) * G; ++e) {
        const float v = s_sel[wave][e];
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
      const unsigned long long key = lane < n_group ? make_key(gscore, lane) : 0ull;
      const int q = key_index(wave_max_u64(key));
      kept |= 1ull << q;
      if (lane == q) gscore = -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((kept >> (e / G)) & 1ull)) val[i] = -INFINITY;
    }
  }
  // top-k by repeated 64-lane argmax
  int my_idx = 0;
  for (int j = 0; j < k; ++j) {
    unsigned long long best = 0;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + 64 * i;
      if (e < E) {
        const unsigned long long key = make_key(val[i], e);
        best = key > best ? key : best;
      }
    }
    const int e = key_index(wave_max_u64(best));
    if (lane == j) my_idx = e;
    if (lane == (e & 63)) {
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i)
        if (i == (e >> 6)) val[i] = -INFINITY;
    }
  }
  // normalize the unbiased scores of the chosen experts, then scale
  float sum = 0.f;
  for (int j = 0; j < k; ++j) {
    const int e = __shfl(my_idx, j, 64);
    sum += s_sc[wave][e];
  }
  if (lane < k) {
    const float w = s_sc[wave][my_idx] / sum;
    topk_idx[static_cast<int64_t>(t) * k + lane] = my_idx;
    topk_w[static_cast<int64_t>(t) * k + lane] = w * routed_scale;
  }
}

// H split of the router GEMM: S chunks of `chunk` columns (a multiple of 32).
struct Split {
  int S, chunk;
};
bool router_mfma_path(int x_fmt, int H) { return x_fmt == MOE_BF16 && H % kRtK == 0; }

Split router_split(int T, int H, int E, bool mfma) {
  const int64_t tiles =
      mfma ? static_cast<int64_t>((T + kRtTok - 1) / kRtTok) * ((E + kRtExp - 1) / kRtExp)
           : static_cast<int64_t>((T + kTile - 1) / kTile) * ((E + kTile - 1) / kTile);
  const int align = mfma ? kRtK : 32;
  int S = 1;
  if (tiles < kTargetWgs) {
    const int64_t want = (kTargetWgs + tiles - 1) / tiles;
    const int most = std::max(1, H / kMinChunk);
    S = static_cast<int>(std::min<int64_t>(want, most));
  }
  int chunk = (H + S - 1) / S;
  chunk = (chunk + align - 1) / align * align;
  S = (H + chunk - 1) / chunk;
  return {S, chunk};
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_route_workspace(int T, int H, int E) {
  if (T <= 0 || H <= 0 || E <= 0) return 0;
  // the larger of the two paths' needs (the x format is not an argument)
  const Split a = router_split(T, H, E, H % kRtK == 0), b = router_split(T, H, E, false);
  const Split sp = a.S > b.S ? a : b;
  return static_cast<size_t>(sp.S) * T * E * sizeof(float);
}

extern "C" int moe_route(const void* x, int x_fmt, const void* w_router, const float* bias,
                         const float* logits_in, int T, int H, int E, int n_group,
                         int topk_group, int k, float routed_scale, float* logits_out,
                         int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
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
  if (T == 0) return MOE_OK;  // nothing to read or write; pointers may be null
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
  const dim3 sel_grid((T + 3) / 4), block(kThreads);
  if (logits_in) {
    hipLaunchKernelGGL(select_kernel, sel_grid, block, 0, stream, logits_in, 1, bias, T, E,
                       n_group, topk_group, k, routed_scale, logits_out, topk_idx, topk_w);
    return check_launch("moe_route");
  }
  const bool mfma = router_mfma_path(x_fmt, H);
  const Split sp = router_split(T, H, E, mfma);
  const size_t need = static_cast<size_t>(sp.S) * T * E * sizeof(float);
  MOE_REQUIRE(ws && ws_bytes >= need, MOE_ERR_WORKSPACE,
              "moe_route: workspace smaller than moe_route_workspace(T, H, E)");
  float* part = static_cast<float*>(ws);
  if (mfma) {
    const int tiles = ((T + kRtTok - 1) / kRtTok) * ((E + kRtExp - 1) / kRtExp);
    hipLaunchKernelGGL(router_mfma_kernel, dim3(static_cast<unsigned>(tiles * sp.S)), block, 0,
                       stream, static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(w_router), T, H, E, sp.chunk, sp.S, part);
    hipLaunchKernelGGL(select_kernel, sel_grid, block, 0, stream, part, sp.S, bias, T, E, n_group,
                       topk_group, k, routed_scale, logits_out, topk_idx, topk_w);
    return check_launch("moe_route");
  }
  const int tiles = ((T + kTile - 1) / kTile) * ((E + kTile - 1) / kTile);
  const dim3 grid(static_cast<unsigned>(tiles * sp.S));
  if (x_fmt == MOE_BF16)
    hipLaunchKernelGGL(router_gemm_kernel<MOE_BF16>, grid, block, 0, stream, x, w_router, T, H, E,
                       sp.chunk, sp.S, part);
  else
    hipLaunchKernelGGL(router_gemm_kernel<MOE_F32>, grid, block, 0, stream, x, w_router, T, H, E,
                       sp.chunk, sp.S, part);
  hipLaunchKernelGGL(select_kernel, sel_grid, block, 0, stream, part, sp.S, bias, T, E, n_group,
                     topk_group, k, routed_scale, logits_out, topk_idx, topk_w);
  return check_launch("moe_route");
}
