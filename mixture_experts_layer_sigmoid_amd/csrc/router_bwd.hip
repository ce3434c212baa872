// Training steps around the routing: the router backward (combine-weight
// gradient -> score gradient through the normalization -> logit gradient
// through the sigmoid -> input and router-weight gradients), the
// sequence-wise balance loss and the aux-loss-free bias update.
//
// Page "[PyTorch] DeepSeekV3Layer: full MoE transformer layer (MLA +
// DeepSeek MoE)": Description, DeepSeekV3MoE item (sigmoid router with an
// aux-loss-free bias and grouped top-k) and Changes section (optional
// sequence-wise aux loss). The pages give no formula; the rules followed are
// those of DeepSeek-V3:
//   dw[t, j]   = <dOut[t], y[row(t, j)]>
//   ds[t, e_j] = scale / S_t * (dw[t, j] - sum_i dw[t, i] s[t, e_i] / S_t)
//   dlogit     = ds * s * (1 - s)      (selected experts; the selection and
//                                       the bias carry no gradient)
//   balance loss over sequences of L tokens, alpha * mean over sequences of
//   sum_i f_i P_i with f_i = E / (k L) * (tokens selecting i), P_i the mean
//   of s[t, i] / sum_m s[t, m]; its logit gradient
//   (g_m - sum_i g_i s'[t, i]) / Z_t * s (1 - s), g_i = alpha / n_seq f_i / L
//   dx = dlogit . W_r,  dW_r = dlogit^T . x
//   bias update b_i += gamma * sign(T k / E - load_i)
//
// gfx950 design: the per-token step is one wavefront per token (the k dot
// products over H with 16-byte loads, wave reductions); the two GEMMs run on
// bf16 matrix cores (32x32x16) with the logit gradient rounded to bf16 and
// fp32 accumulation, 128 x 128 tiles of four waves, the K-contiguous
// operand staged in LDS as is and the N-contiguous one transposed while it
// is stored to LDS; the long contraction of dW_r (over tokens) is split in
// chunks whose fp32 partial tiles are added in a fixed order.
#include "common.h"
#include "gemm_util.h"

#include <algorithm>
#include <string>

namespace moe {
namespace {

constexpr int kMaxE = 512;
constexpr int kAuxParts = 32;      // token chunks per sequence for the loss statistics
constexpr int kSplitMax = 8;       // contraction chunks of dW_r

__device__ __forceinline__ float sigm(float v) { return 1.f / (1.f + __expf(-v)); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int F>
__device__ __forceinline__ void load8(const void* p, int64_t i, float* v) {
  if constexpr (F == MOE_BF16) {
    const u32x4_t q = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(p) + i);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[2 * c] = __uint_as_float(q[c] << 16);
      v[2 * c + 1] = __uint_as_float(q[c] & 0xFFFF0000u);
    }
  } else {
    load8_f32(static_cast<const float*>(p) + i, v);
  }
}

// ---- balance-loss statistics: per (sequence, token chunk) the expert
// selection counts and the sums of s' = s / sum(s) ----
__global__ __launch_bounds__(256) void aux_partial_kernel(const float* __restrict__ logits,
                                                          const int32_t* __restrict__ idx, int T,
                                                          int k, int E, int L,
                                                          int32_t* __restrict__ cnt_part,
                                                          float* __restrict__ sp_part) {
  __shared__ int32_t s_cnt[kMaxE];
  __shared__ float s_sp[4][kMaxE];
  const int q = blockIdx.x / kAuxParts, part = blockIdx.x % kAuxParts;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += 256) s_cnt[e] = 0;
  for (int e = lane; e < E; e += 64) s_sp[wave][e] = 0.f;
  __syncthreads();
  const int lo = q * L + L * part / kAuxParts, hi = q * L + L * (part + 1) / kAuxParts;
  constexpr int kPer = kMaxE / 64;
  float acc[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) acc[i] = 0.f;
  for (int t = lo + wave; t < hi; t += 4) {
    float sv[kPer];
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = lane + 64 * i;
      sv[i] = e < E ? sigm(logits[static_cast<int64_t>(t) * E + e]) : 0.f;
      z += sv[i];
    }
    z = wave_sum(z);
#pragma unroll
    for (int i = 0; i < kPer; ++i) acc[i] += sv[i] / z;
    if (lane < k) atomicAdd(&s_cnt[idx[static_cast<int64_t>(t) * k + lane]], 1);
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (lane + 64 * i < E) s_sp[wave][lane + 64 * i] = acc[i];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    const int64_t o = static_cast<int64_t>(blockIdx.x) * E + e;
    cnt_part[o] = s_cnt[e];
    sp_part[o] = ((s_sp[0][e] + s_sp[1][e]) + s_sp[2][e]) + s_sp[3][e];
  }
}

// per sequence: f, P, the sequence's sum_i f_i P_i and the gradient weights
// g_i = alpha / n_seq * f_i / L (parts added in a fixed order)
__global__ __launch_bounds__(256) void aux_finish_kernel(const int32_t* __restrict__ cnt_part,
                                                         const float* __restrict__ sp_part, int k,
                                                         int E, int L, int nseq, float alpha,
                                                         float* __restrict__ g,
                                                         float* __restrict__ seq_loss) {
  __shared__ float red[256];
  const int q = blockIdx.x;
  float part = 0.f;
  for (int e = threadIdx.x; e < E; e += 256) {
    int c = 0;
    float sp = 0.f;
    for (int p = 0; p < kAuxParts; ++p) {
      const int64_t o = (static_cast<int64_t>(q) * kAuxParts + p) * E + e;
      c += cnt_part[o];
      sp += sp_part[o];
    }
    const float f = static_cast<float>(E) / (static_cast<float>(k) * L) * c;
    part += f * (sp / L);
    g[static_cast<int64_t>(q) * E + e] = alpha / nseq * f / L;
  }
  red[threadIdx.x] = part;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) seq_loss[q] = red[0];
}

__global__ __launch_bounds__(64) void aux_loss_kernel(const float* __restrict__ seq_loss, int nseq,
                                                      float alpha, float* __restrict__ loss) {
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int q = 0; q < nseq; ++q) s += seq_loss[q];
    *loss = alpha * s / nseq;
  }
}

// ---- per token (one wave): dw, dlogits (+ the balance-loss gradient), the
// bf16 copies of dlogits for the two GEMMs ([T, E] and transposed [E, T]) ----
template <int F>
__global__ __launch_bounds__(256) void route_dlogit_kernel(
    const void* __restrict__ dout, const void* __restrict__ y, const int32_t* __restrict__ row_map,
    const int32_t* __restrict__ idx, const float* __restrict__ logits, int T, int k, int E, int H,
    float scale, const float* __restrict__ g, int L, float* __restrict__ dlogits,
    uint16_t* __restrict__ dl_bf, uint16_t* __restrict__ dlt_bf, int Tp) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tp) return;
  if (t >= T) {            // zero padding columns of the transposed copy
    for (int e = lane; e < E; e += 64) dlt_bf[static_cast<int64_t>(e) * Tp + t] = 0;
    return;
  }
  // dw[j] = <dout[t], y[row(t, j)]>, fp32, 8 values per lane per step
  float dw[16];
  int64_t rows[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    dw[j] = 0.f;
    rows[j] = j < k ? row_map[static_cast<int64_t>(t) * k + j] : 0;
  }
  for (int h = lane * 8; h < H; h += 512) {
    float d[8];
    load8<F>(dout, static_cast<int64_t>(t) * H + h, d);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < k) {
        float v[8];
        load8<F>(y, rows[j] * H + h, v);
#pragma unroll
        for (int q = 0; q < 8; ++q) dw[j] = fmaf(d[q], v[q], dw[j]);
      }
    }
  }
  float ssel[16];
  float S = 0.f, inner = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < k) {
      dw[j] = wave_sum(dw[j]);
      ssel[j] = sigm(logits[static_cast<int64_t>(t) * E + idx[static_cast<int64_t>(t) * k + j]]);
      S += ssel[j];
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j < k) inner += dw[j] * ssel[j];
  inner /= S;
  // balance-loss part for every expert of the token
  constexpr int kPer = kMaxE / 64;
  float sv[kPer], gv[kPer];
  float Z = 0.f, gin = 0.f;
  const float* gq = g ? g + static_cast<int64_t>(t / L) * E : nullptr;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + 64 * i;
    sv[i] = e < E ? sigm(logits[static_cast<int64_t>(t) * E + e]) : 0.f;
    gv[i] = (gq && e < E) ? gq[e] : 0.f;
    Z += sv[i];
    gin += gv[i] * sv[i];
  }
  if (gq) {
    Z = wave_sum(Z);
    gin = wave_sum(gin) / Z;
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + 64 * i;
    if (e >= E) continue;
    float dl = gq ? (gv[i] - gin) / Z * sv[i] * (1.f - sv[i]) : 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < k && idx[static_cast<int64_t>(t) * k + j] == e) {
        const float ds = scale / S * (dw[j] - inner);
        dl += ds * ssel[j] * (1.f - ssel[j]);
      }
    }
    if (dlogits) dlogits[static_cast<int64_t>(t) * E + e] = dl;
    const uint16_t b = f32_to_bf16_bits(dl);
    dl_bf[static_cast<int64_t>(t) * E + e] = b;
    dlt_bf[static_cast<int64_t>(e) * Tp + t] = b;
  }
}

// ---- C[M, N] (+)= A[M, K] . B[K, N], bf16 inputs, fp32 accumulation ----
// A row-major (K contiguous, row stride lda, a multiple of 8), B row-major
// (N contiguous, N a multiple of 8) with rows k >= kvalid_b read as zero. 128 x 128 tiles,
// 4 waves of 64 x 64 (2 x 2 blocks of 32 x 32); K steps of 32 staged in LDS:
// A rows as loaded (64-byte rows, 16-byte chunks XOR-swizzled by row / 4),
// B transposed into [n][k] rows of the same form. blockIdx.y picks the
// contraction chunk [kc * kchunk, +kchunk); chunk kc writes its fp32 tile
// to part + kc * M * N (or, with one chunk and out_bf16, bf16 to out).
constexpr int kGT = 128;
constexpr int kGK = 32;

__global__ __launch_bounds__(256) void gemm_bt_kernel(const uint16_t* __restrict__ A, int lda,
                                                      const uint16_t* __restrict__ B, int kvalid_b,
                                                      int M, int N, int K, int kchunk,
                                                      float* __restrict__ part,
                                                      uint16_t* __restrict__ out_bf16) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[kGT * kGK * 2];
  __shared__ __attribute__((aligned(16))) uint8_t sB[kGT * kGK * 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ntn = (N + kGT - 1) / kGT;
  const int m0 = (blockIdx.x / ntn) * kGT, n0 = (blockIdx.x % ntn) * kGT;
  const int kc = blockIdx.y;
  const int kbeg = kc * kchunk, kend = min(K, kbeg + kchunk);
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};
  const u32x4_t zero4{0u, 0u, 0u, 0u};
  for (int k0 = kbeg; k0 < kend; k0 += kGK) {
    // A: 128 rows x 4 chunks of 8 values; B: 32 k-rows x 16 chunks of 8 n
    u32x4_t ra[2], rb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      const int r = c >> 2, ch = c & 3;
      const int gm = m0 + r, gk = k0 + ch * 8;
      ra[i] = (gm < M && gk < kend) ? *reinterpret_cast<const u32x4_t*>(A + static_cast<int64_t>(gm) * lda + gk)
                                    : zero4;
      const int kr = c >> 4, nch = c & 15;
      const int gk2 = k0 + kr, gn = n0 + nch * 8;
      rb[i] = (gk2 < kend && gk2 < kvalid_b && gn < N)
                  ? *reinterpret_cast<const u32x4_t*>(B + static_cast<int64_t>(gk2) * N + gn)
                  : zero4;
    }
    // the previous step's operand reads are done before the tiles are rewritten
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      const int r = c >> 2, ch = c & 3;
      *reinterpret_cast<u32x4_t*>(sA + swz<64>(r, ch)) = ra[i];
      const int kr = c >> 4, nch = c & 15;
      // 8 consecutive n of k-row kr -> column kr of rows n .. n+7 of [n][k]
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int n = nch * 8 + q;
        const uint16_t v = static_cast<uint16_t>((q & 1) ? (rb[i][q >> 1] >> 16) : (rb[i][q >> 1] & 0xFFFFu));
        *reinterpret_cast<uint16_t*>(sB + swz<64>(n, kr >> 3) + (kr & 7) * 2) = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kGK / 16; ++s) {
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 64 * wm + 32 * i + (lane & 31);
        af[i] = *reinterpret_cast<const bf16x8_t*>(sA + swz<64>(r, 2 * s + (lane >> 5)));
        const int n = 64 * wn + 32 * i + (lane & 31);
        bfr[i] = *reinterpret_cast<const bf16x8_t*>(sB + swz<64>(n, 2 * s + (lane >> 5)));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }
  // C layout of a 32x32 MFMA: lane l, element r -> row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = n0 + 64 * wn + 32 * j + (lane & 31);
        if (row < M && col < N) {
          const int64_t o = static_cast<int64_t>(row) * N + col;
          if (out_bf16) out_bf16[o] = f32_to_bf16_bits(acc[i][j][r]);
          else part[static_cast<int64_t>(kc) * M * N + o] = acc[i][j][r];
        }
      }
}

// out[i] = sum over chunks c (in order) of part[c][i], fp32 or bf16 out
__global__ __launch_bounds__(256) void sum_parts_kernel(const float* __restrict__ part, int nparts,
                                                        int64_t n, float* __restrict__ out_f32,
                                                        uint16_t* __restrict__ out_bf16) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += 256ll * gridDim.x) {
    float s = 0.f;
    for (int c = 0; c < nparts; ++c) s += part[c * n + i];
    if (out_f32) out_f32[i] = s;
    else out_bf16[i] = f32_to_bf16_bits(s);
  }
}

__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ counts, int E,
                                                          float gamma, const float* __restrict__ b,
                                                          float* __restrict__ out) {
  __shared__ long long red[256];
  long long s = 0;
  for (int e = threadIdx.x; e < E; e += 256) s += counts[e];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const long long total = red[0];
  for (int e = threadIdx.x; e < E; e += 256) {
    const long long d = total - static_cast<long long>(E) * counts[e];   // sign(mean - load)
    const float sg = d > 0 ? 1.f : (d < 0 ? -1.f : 0.f);
    out[e] = b[e] + gamma * sg;
  }
}

size_t up256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

int dw_split(int T) { return std::max(1, std::min(kSplitMax, T / 512)); }

int pad8(int T) { return (T + 7) / 8 * 8; }

struct RbLayout {
  size_t dl, dlt, part, cnt, sp, g, seql, total;
};

RbLayout rb_layout(int T, int H, int E, int seq_len) {
  RbLayout L{};
  size_t o = 0;
  auto take = [&](size_t b) {
    const size_t at = o;
    o += up256(b);
    return at;
  };
  L.dl = take(static_cast<size_t>(T) * E * 2);
  L.dlt = take(static_cast<size_t>(pad8(T)) * E * 2);
  L.part = take(static_cast<size_t>(dw_split(T)) * E * H * 4);
  const int nseq = seq_len > 0 ? T / seq_len : 0;
  L.cnt = take(static_cast<size_t>(nseq) * kAuxParts * E * 4);
  L.sp = take(static_cast<size_t>(nseq) * kAuxParts * E * 4);
  L.g = take(static_cast<size_t>(nseq) * E * 4);
  L.seql = take(static_cast<size_t>(nseq) * 4);
  L.total = o;
  return L;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_route_bwd_workspace(int T, int H, int E, int seq_len) {
  if (T < 1 || H < 1 || E < 1 || E > kMaxE || seq_len < 0 || (seq_len > 0 && T % seq_len)) return 0;
  return rb_layout(T, H, E, seq_len).total;
}

extern "C" int moe_route_bwd(const void* dout, const void* y, int act_fmt, const int32_t* row_map,
                             const int32_t* topk_idx, const float* logits, const void* x,
                             const void* w_router, int T, int k, int E, int H, float routed_scale,
                             int seq_len, float aux_alpha, float* dlogits, float* aux_loss,
                             void* dx_router, float* dw_router, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(T >= 0 && k >= 1 && k <= 16 && E >= 8 && E <= kMaxE && E % 8 == 0 && k <= E &&
                  H > 0 && H % 8 == 0,
              MOE_ERR_INVALID_ARG,
              "moe_route_bwd: need T >= 0, 1 <= k <= min(16, E), E a multiple of 8 in [8, 512], H "
              "a positive multiple of 8");
  MOE_REQUIRE(act_fmt == MOE_BF16, MOE_ERR_UNSUPPORTED,
              "moe_route_bwd: act_fmt (dout, y, x, w_router, dx_router) must be MOE_BF16");
  const bool aux = aux_alpha != 0.f;
  MOE_REQUIRE(!aux || (seq_len > 0 && T % seq_len == 0), MOE_ERR_INVALID_ARG,
              "moe_route_bwd: the balance loss needs seq_len > 0 dividing T");
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(dout && y && row_map && topk_idx && logits && x && w_router && dx_router &&
                  dw_router && (!aux || aux_loss),
              MOE_ERR_INVALID_ARG, "moe_route_bwd: null pointer");
  MOE_REQUIRE(aligned16(dout) && aligned16(y) && aligned16(x) && aligned16(w_router),
              MOE_ERR_ALIGNMENT, "moe_route_bwd: dout, y, x and w_router must be 16-byte aligned");
  const RbLayout Lo = rb_layout(T, H, E, aux ? seq_len : 0);
  MOE_REQUIRE(ws && ws_bytes >= Lo.total && aligned16(ws), MOE_ERR_WORKSPACE,
              "moe_route_bwd: workspace missing, unaligned or smaller than "
              "moe_route_bwd_workspace(T, H, E, seq_len) = " + std::to_string(Lo.total) + " bytes");
  uint8_t* w = static_cast<uint8_t*>(ws);
  uint16_t* dl_bf = reinterpret_cast<uint16_t*>(w + Lo.dl);
  uint16_t* dlt_bf = reinterpret_cast<uint16_t*>(w + Lo.dlt);
  float* part = reinterpret_cast<float*>(w + Lo.part);
  float* g = nullptr;
  if (aux) {
    const int nseq = T / seq_len;
    int32_t* cnt = reinterpret_cast<int32_t*>(w + Lo.cnt);
    float* sp = reinterpret_cast<float*>(w + Lo.sp);
    g = reinterpret_cast<float*>(w + Lo.g);
    float* seql = reinterpret_cast<float*>(w + Lo.seql);
    hipLaunchKernelGGL(aux_partial_kernel, dim3(nseq * kAuxParts), dim3(256), 0, stream, logits,
                       topk_idx, T, k, E, seq_len, cnt, sp);
    hipLaunchKernelGGL(aux_finish_kernel, dim3(nseq), dim3(256), 0, stream, cnt, sp, k, E, seq_len,
                       nseq, aux_alpha, g, seql);
    hipLaunchKernelGGL(aux_loss_kernel, dim3(1), dim3(64), 0, stream, seql, nseq, aux_alpha,
                       aux_loss);
  }
  const int Tp = pad8(T);
  hipLaunchKernelGGL(route_dlogit_kernel<MOE_BF16>, dim3((Tp + 3) / 4), dim3(256), 0, stream, dout,
                     y, row_map, topk_idx, logits, T, k, E, H, routed_scale, g,
                     aux ? seq_len : 1, dlogits, dl_bf, dlt_bf, Tp);
  // dx = dlogits . W_r: M = T, N = H, K = E
  const int tiles_dx = ((T + kGT - 1) / kGT) * ((H + kGT - 1) / kGT);
  hipLaunchKernelGGL(gemm_bt_kernel, dim3(tiles_dx, 1), dim3(256), 0, stream, dl_bf, E,
                     static_cast<const uint16_t*>(w_router), E, T, H, E, E, nullptr,
                     static_cast<uint16_t*>(dx_router));
  // dW_r = dlogits^T . x: M = E, N = H, K = tokens (rows of the transposed
  // copy padded to Tp with zeros) in S chunks, added in order
  const int S = dw_split(T);
  const int kchunk = ((Tp + S - 1) / S + kGK - 1) / kGK * kGK;
  const int tiles_dw = ((E + kGT - 1) / kGT) * ((H + kGT - 1) / kGT);
  hipLaunchKernelGGL(gemm_bt_kernel, dim3(tiles_dw, S), dim3(256), 0, stream, dlt_bf, Tp,
                     static_cast<const uint16_t*>(x), T, E, H, Tp, kchunk, part, nullptr);
  const int64_t n = static_cast<int64_t>(E) * H;
  hipLaunchKernelGGL(sum_parts_kernel, dim3(static_cast<unsigned>(std::min<int64_t>(4096, (n + 255) / 256))),
                     dim3(256), 0, stream, part, S, n, dw_router, nullptr);
  return check_launch("moe_route_bwd");
}

extern "C" int moe_bias_update(const int32_t* counts, int E, float gamma, const float* bias,
                               float* bias_out, hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(E >= 1 && E <= 1024, MOE_ERR_INVALID_ARG, "moe_bias_update: need 1 <= E <= 1024");
  MOE_REQUIRE(counts && bias && bias_out, MOE_ERR_INVALID_ARG, "moe_bias_update: null pointer");
  hipLaunchKernelGGL(bias_update_kernel, dim3(1), dim3(256), 0, stream, counts, E, gamma, bias,
                     bias_out);
  return check_launch("moe_bias_update");
}
