// moe_permute: expert-major permutation maps and row gather.
//
// Page "[PyTorch] DeepSeekV3Layer: full MoE transformer layer (MLA +
// DeepSeek MoE)", Performance section, "Where the time goes" table: local
// permute ("dup") of the staging buffer into an expert-major layout with
// zero-filled padding. Rows of one expert follow (token, slot) order, each
// expert segment is padded to a multiple of `align`, padding rows carry
// source -1 and zero bytes.
//
// No atomics anywhere, so every output is deterministic:
//   1. histogram: the T*k (token, slot) entries are cut into chunks of 1024;
//      one wavefront counts its chunk. Lanes holding the same expert find
//      each other with one ballot per index bit; the lowest such lane adds
//      the group's size to the wave's private LDS counter. The kernel also
//      marks every row of src_row as padding (-1).
//   2. scan: one workgroup turns the [chunks, E] histogram into per-chunk
//      row bases (column prefix + padded exclusive scan over experts) and
//      writes counts and offsets; each expert column is split over up to 32
//      threads, whose partial sums are combined in LDS.
//   3. scatter: each wavefront re-walks its chunk in order; an entry's row is
//      its chunk base + running count + number of lower lanes with the same
//      expert, which keeps (token, slot) order. It writes row_map and
//      src_row.
//   4. gather (optional): one workgroup per row copies the source row's
//      bytes with 16-byte loads, or writes zeros for padding rows.
#include "common.h"

#include <algorithm>
#include <mutex>
#include <string>

namespace moe {
namespace {

constexpr int kChunk = 1024;      // entries per wavefront
constexpr int kMaxE = 1024;

__device__ __forceinline__ unsigned long long same_value_lanes(int v, bool valid, int nbits) {
  unsigned long long peers = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (v >> b) & 1;
    const unsigned long long m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ idx, int64_t n,
                                                   int E, int nbits, int nchunks,
                                                   int32_t* __restrict__ hist,
                                                   int32_t* __restrict__ src_row,
                                                   int64_t bound) {
  __shared__ int32_t cnt[4][kMaxE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int64_t r = blockIdx.x * 256ll + threadIdx.x; r < bound; r += 256ll * gridDim.x)
    src_row[r] = -1;
  const int c = blockIdx.x * 4 + wave;
  if (c >= nchunks) return;
  for (int e = lane; e < E; e += 64) cnt[wave][e] = 0;
  wave_lds_sync();
  const int64_t base = static_cast<int64_t>(c) * kChunk;
  // the chunk's indices, all loads in flight at once
  int ev[kChunk / 64];
#pragma unroll
  for (int it = 0; it < kChunk / 64; ++it) {
    const int64_t i = base + 64 * it + lane;
    ev[it] = i < n ? idx[i] : 0;
  }
#pragma unroll
  for (int it = 0; it < kChunk / 64; ++it) {
    const int64_t i = base + 64 * it + lane;
    const bool valid = i < n;
    const int e = ev[it];
    const unsigned long long peers = same_value_lanes(e, valid, nbits);
    if (valid && lane == __ffsll(static_cast<long long>(peers)) - 1)
      cnt[wave][e] += __popcll(peers);
    wave_lds_sync();
  }
  for (int e = lane; e < E; e += 64) hist[static_cast<int64_t>(c) * E + e] = cnt[wave][e];
}

__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ hist, int nchunks, int E,
                                                    int align, int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets) {
  __shared__ int32_t padded[kMaxE];
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  // tpc threads per expert column, each over a contiguous range of chunks
  // (tpc a power of two, tpc * E <= 1024); loads go out eight at a time
  int tpc = 1;
  while (tpc < 32 && 2 * tpc * E <= 1024) tpc <<= 1;
  const int e = tid / tpc, q = tid % tpc;
  const int per = (nchunks + tpc - 1) / tpc;
  const int c_lo = min(nchunks, q * per), c_hi = min(nchunks, c_lo + per);
  const bool col = e < E;
  // pass 1: rows of expert e in this thread's chunks
  int sum = 0;
  if (col) {
    for (int c = c_lo; c < c_hi; c += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = c + u < c_hi ? hist[static_cast<int64_t>(c + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += v[u];
    }
    part[tid] = sum;
  }
  __syncthreads();
  // counts and padded counts per expert
  for (int x = tid; x < E; x += 1024) {
    int run = 0;
    for (int r = 0; r < tpc; ++r) run += part[x * tpc + r];
    counts[x] = run;
    padded[x] = (run + align - 1) / align * align;
  }
  __syncthreads();
  // exclusive scan of the padded counts: each thread sums a contiguous run
  // of experts, then the 1024 partial sums are scanned in LDS (part[] is
  // read into registers first: it is reused here)
  int before = 0;  // rows of expert e in the chunks before this thread's
  if (col)
    for (int r = 0; r < q; ++r) before += part[e * tpc + r];
  __syncthreads();
  const int pe = (E + 1023) / 1024;
  const int lo = tid * pe, hi = min(E, lo + pe);
  int s = 0;
  for (int x = lo; x < hi; ++x) s += padded[x];
  part[tid] = s;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int v = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = tid > 0 ? part[tid - 1] : 0;
  for (int x = lo; x < hi; ++x) {
    const int p = padded[x];
    padded[x] = run;  // becomes the exclusive offset
    run += p;
  }
  if (tid == 1023) offsets[E] = part[1023];
  __syncthreads();
  for (int x = tid; x < E; x += 1024) offsets[x] = padded[x];
  // pass 2: hist[c][e] becomes the first row of expert e's entries of chunk
  // c: the expert's offset plus its rows in the chunks before c
  if (col) {
    int r0 = padded[e] + before;
    for (int c = c_lo; c < c_hi; c += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = c + u < c_hi ? hist[static_cast<int64_t>(c + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (c + u < c_hi) hist[static_cast<int64_t>(c + u) * E + e] = r0;
        r0 += v[u];
      }
    }
  }
}

__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ idx, int64_t n,
                                                      int k, int E, int nbits, int nchunks,
                                                      const int32_t* __restrict__ base_rows,
                                                      int32_t* __restrict__ row_map,
                                                      int32_t* __restrict__ src_row) {
  __shared__ int32_t run[4][kMaxE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.x * 4 + wave;
  if (c >= nchunks) return;
  for (int e = lane; e < E; e += 64) run[wave][e] = base_rows[static_cast<int64_t>(c) * E + e];
  wave_lds_sync();
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t base = static_cast<int64_t>(c) * kChunk;
  int ev[kChunk / 64];
#pragma unroll
  for (int it = 0; it < kChunk / 64; ++it) {
    const int64_t i = base + 64 * it + lane;
    ev[it] = i < n ? idx[i] : 0;
  }
#pragma unroll
  for (int it = 0; it < kChunk / 64; ++it) {
    const int64_t i = base + 64 * it + lane;
    const bool valid = i < n;
    const int e = ev[it];
    const unsigned long long peers = same_value_lanes(e, valid, nbits);
    int row = 0;
    if (valid) row = run[wave][e] + __popcll(peers & below);
    wave_lds_sync();
    if (valid && lane == __ffsll(static_cast<long long>(peers)) - 1)
      run[wave][e] += __popcll(peers);
    wave_lds_sync();
    if (valid) {
      row_map[i] = row;
      src_row[row] = static_cast<int32_t>(i / k);
    }
  }
}

__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* __restrict__ in,
                                                          int64_t row_bytes,
                                                          const int32_t* __restrict__ src_row,
                                                          int64_t bound, uint8_t* __restrict__ out) {
  const int64_t nvec = row_bytes / 16;
  for (int64_t r = blockIdx.x; r < bound; r += gridDim.x) {
    const int s = src_row[r];
    u32x4_t* o = reinterpret_cast<u32x4_t*>(out + r * row_bytes);
    if (s < 0) {
      for (int64_t v = threadIdx.x; v < nvec; v += 256) o[v] = u32x4_t{0u, 0u, 0u, 0u};
    } else {
      const u32x4_t* p = reinterpret_cast<const u32x4_t*>(in + static_cast<int64_t>(s) * row_bytes);
      for (int64_t v = threadIdx.x; v < nvec; v += 256) o[v] = p[v];
    }
  }
}

__global__ __launch_bounds__(256) void gather_bytes_kernel(const uint8_t* __restrict__ in,
                                                           int64_t row_bytes,
                                                           const int32_t* __restrict__ src_row,
                                                           int64_t bound, uint8_t* __restrict__ out) {
  const int64_t total = bound * row_bytes;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < total; i += 256ll * gridDim.x) {
    const int64_t r = i / row_bytes, b = i % row_bytes;
    const int s = src_row[r];
    out[i] = s < 0 ? 0 : in[static_cast<int64_t>(s) * row_bytes + b];
  }
}

int nchunks_of(int64_t n) { return static_cast<int>(n > 0 ? (n + kChunk - 1) / kChunk : 1); }

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int64_t moe_permute_rows_bound(int T, int k, int E, int align) {
  if (T < 0 || k < 1 || E < 1 || align < 1) return -1;
  return static_cast<int64_t>(T) * k + static_cast<int64_t>(E) * (align - 1);
}

extern "C" size_t moe_permute_workspace(int T, int k, int E) {
  if (T < 0 || k < 1 || E < 1) return 0;
  return static_cast<size_t>(nchunks_of(static_cast<int64_t>(T) * k)) * E * sizeof(int32_t);
}

// Argument checks shared by moe_permute and moe_permute_noalloc (everything
// but the workspace).
static int check_permute(const char* fn, const int32_t* topk_idx, int T, int k, int E, int align,
                         const void* rows_in, int64_t row_bytes, const void* scales_in,
                         int64_t scale_bytes, int32_t* counts, int32_t* offsets, int32_t* row_map,
                         int32_t* src_row, void* rows_out, void* scales_out) {
  const std::string f(fn);
  MOE_REQUIRE(T >= 0 && k >= 1 && E >= 1 && E <= kMaxE, MOE_ERR_INVALID_ARG,
              f + ": need T >= 0, k >= 1, 1 <= E <= 1024");
  MOE_REQUIRE(align == 1 || align == 16 || align == 32 || align == 64 || align == 128,
              MOE_ERR_INVALID_ARG, f + ": align must be 1, 16, 32, 64 or 128");
  MOE_REQUIRE(static_cast<int64_t>(T) * k + static_cast<int64_t>(E) * align < (1ll << 31),
              MOE_ERR_INVALID_ARG, f + ": row count exceeds int32");
  MOE_REQUIRE(counts && offsets && src_row && (T == 0 || (topk_idx && row_map)),
              MOE_ERR_INVALID_ARG, f + ": null map pointer");
  MOE_REQUIRE((rows_in == nullptr) == (rows_out == nullptr), MOE_ERR_INVALID_ARG,
              f + ": rows_in and rows_out go together");
  MOE_REQUIRE((scales_in == nullptr) == (scales_out == nullptr), MOE_ERR_INVALID_ARG,
              f + ": scales_in and scales_out go together");
  if (rows_in) {
    MOE_REQUIRE(row_bytes > 0, MOE_ERR_INVALID_ARG, f + ": row_bytes must be > 0");
    MOE_REQUIRE(row_bytes % 16 == 0 && aligned16(rows_in) && aligned16(rows_out),
                MOE_ERR_ALIGNMENT, f + ": rows and row_bytes must be 16-byte aligned");
  }
  if (scales_in)
    MOE_REQUIRE(scale_bytes > 0, MOE_ERR_INVALID_ARG, f + ": scale_bytes must be > 0");
  return MOE_OK;
}

// The permutation's kernels on a histogram buffer `hist` of at least
// moe_permute_workspace(T, k, E) bytes (fully written by the first kernel
// before it is read, so its previous contents do not matter).
static int permute_launch(const int32_t* topk_idx, int T, int k, int E, int align,
                          const void* rows_in, int64_t row_bytes, const void* scales_in,
                          int64_t scale_bytes, int32_t* counts, int32_t* offsets,
                          int32_t* row_map, int32_t* src_row, void* rows_out, void* scales_out,
                          int32_t* hist, hipStream_t stream, const char* fn) {
  const int64_t n = static_cast<int64_t>(T) * k;
  const int nchunks = nchunks_of(n);
  const int64_t bound = moe_permute_rows_bound(T, k, E, align);
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int hgrid = std::max<int64_t>((nchunks + 3) / 4, std::min<int64_t>(1024, (bound + 255) / 256));
  hipLaunchKernelGGL(hist_kernel, dim3(hgrid), dim3(256), 0, stream, topk_idx, n, E, nbits,
                     nchunks, hist, src_row, bound);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, stream, hist, nchunks, E, align, counts,
                     offsets);
  if (n > 0)
    hipLaunchKernelGGL(scatter_kernel, dim3((nchunks + 3) / 4), dim3(256), 0, stream, topk_idx, n,
                       k, E, nbits, nchunks, hist, row_map, src_row);
  if (rows_in && bound > 0)
    hipLaunchKernelGGL(gather_rows_kernel, dim3(static_cast<unsigned>(std::min<int64_t>(bound, 8192))),
                       dim3(256), 0, stream, static_cast<const uint8_t*>(rows_in), row_bytes,
                       src_row, bound, static_cast<uint8_t*>(rows_out));
  if (scales_in && bound > 0) {
    const int64_t g = std::min<int64_t>(8192, (bound * scale_bytes + 255) / 256);
    hipLaunchKernelGGL(gather_bytes_kernel, dim3(static_cast<unsigned>(g)), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(scales_in), scale_bytes, src_row, bound,
                       static_cast<uint8_t*>(scales_out));
  }
  return check_launch(fn);
}

extern "C" int moe_permute(const int32_t* topk_idx, int T, int k, int E, int align,
                           const void* rows_in, int64_t row_bytes, const void* scales_in,
                           int64_t scale_bytes, int32_t* counts, int32_t* offsets,
                           int32_t* row_map, int32_t* src_row, void* rows_out, void* scales_out,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  int st = check_permute("moe_permute", topk_idx, T, k, E, align, rows_in, row_bytes, scales_in,
                         scale_bytes, counts, offsets, row_map, src_row, rows_out, scales_out);
  if (st) return st;
  const size_t need = moe_permute_workspace(T, k, E);
  MOE_REQUIRE(ws && ws_bytes >= need, MOE_ERR_WORKSPACE, "moe_permute: workspace too small");
  return permute_launch(topk_idx, T, k, E, align, rows_in, row_bytes, scales_in, scale_bytes,
                        counts, offsets, row_map, src_row, rows_out, scales_out,
                        static_cast<int32_t*>(ws), stream, "moe_permute");
}

// ---- moe_permute_noalloc: the histogram in a file-scope device array ----
// Each GPU the library runs on holds its own copy of `scratch` (1 MiB) until
// the process ends. Host code never passes the array's name to a kernel (in
// host code it is a stand-in, not a device address): the device address is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and kept.
static constexpr size_t kNoAllocScratchBytes = size_t{1} << 20;
static __device__ __align__(256) int32_t scratch[kNoAllocScratchBytes / sizeof(int32_t)];

namespace moe {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};

// device address of `scratch` on the current device (looked up on the first
// call on that device), or null with an error set
int32_t* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    set_error("moe_permute_noalloc: no current HIP device (or device index >= 64)");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      set_error(std::string("moe_permute_noalloc: hipGetSymbolAddress(scratch) failed: ") +
                hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = static_cast<int32_t*>(ptr);
  }
  return g_scratch_ptr[dev];
}
}  // namespace
}  // namespace moe

extern "C" size_t moe_permute_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

extern "C" int moe_permute_noalloc(const int32_t* topk_idx, int T, int k, int E, int align,
                                   const void* rows_in, int64_t row_bytes, const void* scales_in,
                                   int64_t scale_bytes, int32_t* counts, int32_t* offsets,
                                   int32_t* row_map, int32_t* src_row, void* rows_out,
                                   void* scales_out, hipStream_t stream) {
  clear_error();
  int st = check_permute("moe_permute_noalloc", topk_idx, T, k, E, align, rows_in, row_bytes,
                         scales_in, scale_bytes, counts, offsets, row_map, src_row, rows_out,
                         scales_out);
  if (st) return st;
  const size_t need = moe_permute_workspace(T, k, E);
  MOE_REQUIRE(need <= kNoAllocScratchBytes, MOE_ERR_WORKSPACE,
              "moe_permute_noalloc: T * k and E need " + std::to_string(need) +
                  " bytes of histogram, above its fixed 1 MiB (ceil(T * k / 1024) * E * 4 must "
                  "not exceed 1048576); use moe_permute with a workspace");
  int32_t* hist = scratch_on_current_device();
  if (!hist) return MOE_ERR_HIP;
  return permute_launch(topk_idx, T, k, E, align, rows_in, row_bytes, scales_in, scale_bytes,
                        counts, offsets, row_map, src_row, rows_out, scales_out, hist, stream,
                        "moe_permute_noalloc");
}
