// Grouped expert GEMMs over expert-major row segments with weights streamed
// straight into registers: routed fc1 + SwiGLU, fc2, and the data-gradient
// GEMMs of the backward (fc2 dgrad fused with the SwiGLU backward, fc1
// dgrad).
//
// Page "[PyTorch] DeepSeekV3Layer: full MoE transformer layer (MLA +
// DeepSeek MoE)": Description (experts as GroupedLinear -> ScaledSwiGLU ->
// GroupedLinear, fused into one grouped MLP) and Performance section ("Where
// the time goes": fc1+SwiGLU fwd, fc2 fwd and dGLU bwd of the fused grouped
// MLP, MXFP8). Page "Mistral Large 3 NVFP4 TRTLLM MoE support", Highlights:
// fc1's weight holds the w1 (gate) and w3 (up) halves; here rows [0, F) gate,
// [F, 2F) up.
//
// Design (gfx950). At the shapes of these layers the grouped GEMMs stream
// far more weight bytes than activation bytes (a few hundred rows per expert
// against 2F x H weights), so the kernel is built around reading every
// weight byte from HBM once, contiguously, with as much in flight as
// possible:
//   * Weights are packed once (moe_pack_weights) into the order the 32x32
//     MFMA consumes them: for every 32-row column block and every 128 bytes
//     of K ("stage"), 4 KB holding, piece by piece, exactly the 16 bytes
//     each of the 64 lanes feeds its matrix instruction. A wavefront streams
//     its column blocks with plain 16-byte-per-lane loads of contiguous
//     1 KB pieces into a ring of P stages of registers; no LDS, no barrier
//     and no sharing is involved on the weight side. MX block scales are
//     packed the same way (the bytes of one lane's scales for one stage are
//     adjacent).
//   * A tile is (expert e, column tile of 256 weight rows, up to 256 rows of
//     the expert's segment): an expert with at most 256 rows reads its
//     weights exactly once; longer segments are cut into balanced row tiles
//     that run side by side on one XCD, so the second read hits L2. Four
//     wavefronts, one per SIMD; wavefront w owns two column blocks (64
//     weight rows) and every row block of the tile: 16 accumulators of
//     32x32 fp32 in the accumulation registers.
//   * Activation rows are shared by the four wavefronts: they go through a
//     ring of P LDS stages with direct global->LDS 16-byte loads (row
//     gather through src_row for fc1), XOR-swizzled so the MFMA operand
//     reads are free of bank conflicts; the MX scales of the rows ride in
//     small per-stage arrays.
//   * The tile list (experts x column tiles x row tiles) is built in LDS
//     from `offsets` by every workgroup, cut into 8 contiguous chunks, one
//     per XCD; consecutive tiles are the row tiles of one weight tile, then
//     the column tiles of one expert (a long segment in groups of 4 row
//     tiles), so concurrent workgroups of an XCD share activation rows and
//     weight tiles in its L2.
//   * Epilogues go through LDS in passes of 128 rows to row-major 16-byte
//     stores (fc2 and the fc1 data gradient store rows straight from
//     registers): SwiGLU (bf16 h, or MX-encoded 32-column blocks of h formed in
//     registers when the fp32 fc1 output is not saved: a wave holds both
//     halves of the same columns), plain bf16 y, or the SwiGLU backward (dA
//     in MX or bf16, optional fp32 copy).
#include "common.h"
#include "expert_gemm.h"
#include "gemm_util.h"
#include "mx_codec.h"
#include "nvfp4_codec.h"

#include <algorithm>
#include <string>
#include <type_traits>

namespace moe {
namespace {

constexpr int kMaxGroups = 1024;
constexpr int kStageBytes = 128;        // bytes of K per row per stage
constexpr int kPiece = 1024;            // one 16-byte-per-lane weight load
constexpr int kTileCols = 256;          // weight rows per tile (8 column blocks)
constexpr int kCs = kTileCols + 4;      // padded fp32 row stride of the epilogue tile
// Scheduling cost of a tile = kTileCost + its rows: streaming a tile's
// weights takes about as long as the matrix work of ~220 rows at the
// chip's byte-to-flop ratio (the same for bf16, E4M3 and E2M1 tiles).
constexpr int kTileCost = 220;
// A dense expert enters the tile list as kDenseParts row ranges spread
// evenly among the routed experts, so every XCD runs a share of its
// compute-bound tiles beside its share of the weight stream.
constexpr int kDenseParts = 8;
// row tiles per group in the tile order of a long segment
constexpr int kRowGroup = 4;
constexpr int kMaxVirt = kMaxGroups + kDenseParts;

enum { XOP_BF16 = 0, XOP_FP8 = 1, XOP_FP4 = 2, XOP_NVFP4 = 3 };
enum { XEPI_SWIGLU = 0, XEPI_PLAIN = 1, XEPI_DSWIGLU = 2 };

// Per operand format: k-steps of one stage (128 bytes of the activation
// row), MX scale bytes of an activation row per stage, 1 KB weight loads per
// column block and stage, packed weight-scale bytes per (column block,
// stage). XOP_NVFP4: bf16 activation values (code * scale) against E2M1
// weights with E4M3 scales per 16, converted to bf16 in registers (a stage
// is 64 values: 32 bytes of codes per weight row, one 1 KB load).
template <int OP>
struct XOp {
  static constexpr bool kBf16A = OP == XOP_BF16 || OP == XOP_NVFP4;
  static constexpr int kSub = OP == XOP_FP8 ? 2 : 4;
  static constexpr int kScaleBytes = kBf16A ? 0 : (OP == XOP_FP8 ? 4 : 8);
  static constexpr int kPieces = OP == XOP_NVFP4 ? 1 : 4;
  static constexpr int kChunkW = kPieces * kPiece;                        // per (cb, stage)
  // packed weight-scale bytes per (cb, stage): one byte per row and MX block
  // (the two lane halves read different blocks); NVFP4 4 bytes per row, the
  // same word for both lane halves (a k-step is one 16-block)
  static constexpr int kPackedScaleBytes = OP == XOP_BF16 ? 0 : (OP == XOP_NVFP4 ? 128 : 64 * kSub);
  static constexpr int kBLoads = 2 * kPieces + (OP == XOP_BF16 ? 0 : 2);   // per wave and stage
};

struct XArgs {
  const uint8_t* a;          // activation rows [rows, K] (or token rows with gather)
  int64_t a_row_bytes;
  const uint8_t* a_sc;       // their MX scales [rows, K/32]
  int64_t a_sc_row_bytes;
  uint32_t a_bytes;          // bytes of the activation matrix (< 4 GiB) and of its scales
  uint32_t a_sc_bytes;
  const int32_t* gather;     // optional row -> token row (-1: padding row)
  const uint8_t* b;          // packed weights of expert 0
  int64_t b_exp_bytes;
  const uint8_t* b_sc;       // packed MX scales of expert 0
  int64_t b_sc_exp_bytes;
  int ncb;                   // 32-row column blocks per expert (N / 32)
  int n_tiles;               // column tiles per expert (ceil(N / 256))
  int k_stages;              // K bytes / 128
  const int32_t* offsets;    // [E+1]
  int E;
  int64_t rows;
  int half;                  // SwiGLU: F; dSwiGLU: F (offset of the up half)
  uint8_t* out;
  int64_t out_row_bytes;
  uint8_t* out_sc;
  int64_t out_sc_row_bytes;
  float* act_save;           // fc1: optional fp32 [rows, 2F]
  const float* a_saved;      // dSwiGLU: saved fc1 output [rows, 2F] fp32
  float* da_f32;             // dSwiGLU: optional fp32 copy of dA [rows, 2F]
  // NVFP4: tensor scale of the activations, per-expert tensor scales of the
  // weights (applied to the fp32 accumulators) and of the output h (fc1)
  float a_g;
  const float* w_g;
  float out_g;
  // optional dense expert (the shared expert) run by the same launch: it
  // takes d_rows rows, A rows d_a_row0.. and output rows d_row0.., packed
  // weights d_b / d_b_sc; null d_b: none
  const uint8_t* d_b;
  const uint8_t* d_b_sc;
  int d_rows;
  int d_row0;
  int d_a_row0;
};

// epilogue rows per LDS pass: 128, or 64 with two workgroups per CU
template <int OCC>
struct XPass {
  static constexpr int kRows = OCC == 1 ? 128 : 64;
};

template <int MAXNV, int P, int OP, int OCC>
struct XSmem {
  static constexpr int kPassRows = XPass<OCC>::kRows;
  static constexpr int kRows = 32 * MAXNV;
  static constexpr int kA = kRows * kStageBytes;
  static constexpr int kASc = kRows * XOp<OP>::kScaleBytes;
  static constexpr int kStage = kA + kASc;
  static constexpr int kRing = P * kStage;
  static constexpr int kEpi = (kRows < kPassRows ? kRows : kPassRows) * kCs * 4;
  static constexpr int kBody = kRing > kEpi ? kRing : kEpi;
  static constexpr int kSched = (kMaxVirt + 2) * 4 + kRows * 4 + (kMaxVirt + 1) * 4 + kMaxVirt * 2 +
                                (kMaxGroups + 1) * 4;
  static constexpr int kTotal = kBody + kSched;
};

__device__ __forceinline__ float sigmoidf_(float g) { return 1.f / (1.f + expf(-g)); }

// f(integral_constant<0>) ... f(integral_constant<N-1>), unrolled at compile time
template <int I, int N, typename Fn>
__device__ __forceinline__ void static_for_impl(Fn&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, typename Fn>
__device__ __forceinline__ void static_for(Fn&& f) { static_for_impl<0, N>(f); }

// MAXNV: row blocks of 32 per tile (tile rows = 32 * MAXNV)
// P:     stages in flight (LDS ring for the activations, register ring for
//        the weights)
// OCC:   workgroups resident per CU (persistent grid = 256 * OCC)
template <int MAXNV, int P, int OCC, int OP, int EPI, int OUTF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void expert_gemm_kernel(XArgs p) {
  using S = XSmem<MAXNV, P, OP, OCC>;
  constexpr int kPassRows = S::kPassRows;
  using O = XOp<OP>;
  constexpr int kRows = S::kRows;
  constexpr int kSB = O::kScaleBytes;
  constexpr int kSub = O::kSub;
  constexpr int kAIns = kRows / 8 / 4;              // 1 KB A loads per wave per stage (max)
  constexpr int kDpr = kSB > 0 ? kSB / 4 : 1;       // scale dwords per row per stage
  constexpr int kScRows = 64 / kDpr;                // rows per 4-byte-per-lane scale load
  constexpr int kAScIns = kSB > 0 ? (kRows + kScRows - 1) / kScRows : 0;
  // every wave issues the same number of scale loads; when there are fewer
  // loads than waves the extra waves repeat the last one (same bytes to the
  // same LDS words)
  constexpr int kAScPerWave = kSB > 0 ? (kAScIns + 3) / 4 : 0;
  static_assert(kAIns >= 1, "tile needs at least 32 rows");
  // Plain epilogue (bf16 rows out): the weights are the matrix
  // instructions' first operand and the activation rows the second, so the
  // accumulators hold, per lane, one row and 16 of its columns; rows are
  // written straight from registers, with no LDS round trip.
  constexpr bool kRowsInLanes = EPI == XEPI_PLAIN;
  __shared__ __attribute__((aligned(16))) uint8_t smem[S::kTotal];
  int32_t* s_mt = reinterpret_cast<int32_t*>(smem + S::kBody);   // [V+1] row-tile prefix
  int32_t* s_src = s_mt + (kMaxVirt + 1);                         // [kRows] source rows
  int32_t* s_tot = s_src + kRows;
  int32_t* s_cost = s_tot + 1;                                    // [V+1] cost prefix
  int16_t* s_vmap = reinterpret_cast<int16_t*>(s_cost + kMaxVirt + 1);  // [V] -> expert / E + part
  int32_t* s_off = reinterpret_cast<int32_t*>(s_vmap + kMaxVirt);       // [E+1] segment offsets
  int32_t* part = reinterpret_cast<int32_t*>(smem);  // scan scratch (before any load)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int E = p.E;

  // ---- virtual experts: the routed experts in order, with the dense
  // expert's part x after routed expert floor((x+1) E / 8) - 1 ----
  const bool dense = p.d_b != nullptr;
  const int V = E + (dense ? kDenseParts : 0);
  for (int e = tid; e < E; e += 256) {
    int x = 0;
    if (dense)
      while ((x + 1) * E / kDenseParts <= e) ++x;
    s_vmap[e + x] = static_cast<int16_t>(e);
  }
  if (dense && tid < kDenseParts) s_vmap[(tid + 1) * E / kDenseParts + tid] = static_cast<int16_t>(E + tid);
  // the segment offsets, read from LDS by every tile's set-up (no global
  // memory round trip per tile)
  for (int e = tid; e <= E; e += 256) s_off[e] = p.offsets[e];
  __syncthreads();
  // rows of virtual expert v (a routed segment, or a part of the dense rows)
  auto vrows = [&](int v) {
    const int e = s_vmap[v];
    if (e >= E) {
      const int x = e - E;
      return p.d_rows * (x + 1) / kDenseParts - p.d_rows * x / kDenseParts;
    }
    const int n_e = min(s_off[e + 1], (int)p.rows) - s_off[e];
    return n_e < 0 ? 0 : n_e;
  };

  // ---- tile list: row tiles per virtual expert, prefix in s_mt[1..V] ----
  {
    const int per = (V + 255) / 256;
    const int lo = min(V, tid * per), hi = min(V, lo + per);
    int s = 0;
    for (int v = lo; v < hi; ++v) {
      const int mt = (vrows(v) + kRows - 1) / kRows;
      s_mt[v + 1] = mt;
      s += mt;
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
    for (int v = lo; v < hi; ++v) {
      run += s_mt[v + 1];
      s_mt[v + 1] = run;
    }
    if (tid == 0) {
      s_mt[0] = 0;
      s_tot[0] = part[255];
    }
    __syncthreads();
    // cost of an expert's tiles per column tile: every row tile streams the
    // same weight bytes (kTileCost, in the matrix time of that many rows)
    // and does matrix work in proportion to its rows
    int c = 0;
    for (int v = lo; v < hi; ++v) {
      s_cost[v + 1] = (s_mt[v + 1] - s_mt[v]) * kTileCost + vrows(v);
      c += s_cost[v + 1];
    }
    part[tid] = c;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
      const int v = tid >= d ? part[tid - d] : 0;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    run = tid > 0 ? part[tid - 1] : 0;
    for (int v = lo; v < hi; ++v) {
      run += s_cost[v + 1];
      s_cost[v + 1] = run;
    }
    if (tid == 0) s_cost[0] = 0;
    __syncthreads();
  }
  // XCD x runs the tiles between the points where the running cost reaches
  // x/8 and (x+1)/8 of the total (inside an expert, its tiles are taken as
  // equally costly): a skewed routing's long segments, whose row tiles do
  // most of the matrix work, do not pile up on one XCD
  const int64_t total_tiles = static_cast<int64_t>(s_tot[0]) * p.n_tiles;
  const XcdSlot xs = xcd_slot();
  auto boundary = [&](int x) -> int64_t {
    if (x == 0) return 0;
    if (x == kNumXcd) return total_tiles;
    const int64_t target = static_cast<int64_t>(s_cost[V]) * x / kNumXcd;
    int lo = 0, hi = V;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_cost[mid] <= target) lo = mid;
      else hi = mid;
    }
    const int64_t ce = s_cost[lo + 1] - s_cost[lo];
    const int64_t tiles_e = static_cast<int64_t>(s_mt[lo + 1] - s_mt[lo]) * p.n_tiles;
    const int64_t within = ce > 0 ? (target - s_cost[lo]) * tiles_e / ce : 0;
    return static_cast<int64_t>(s_mt[lo]) * p.n_tiles + within;
  };
  const int64_t t_first = boundary(xs.xcd) + xs.slot;
  const int64_t t_end = boundary(xs.xcd + 1);

  // Per-lane LDS offsets of the activation operands inside one stage tile:
  // chunk 2q + g (16 bytes; q = k-step for bf16 / E2M1, 2 k-step + half for
  // E4M3) of row lane % 32 of row block 0, in the swizzled layout (the key
  // depends on row % 16 only, so row block i adds 4 KB), and the row's MX
  // scale words. Every step re-derives its slot's addresses from these
  // (opaque copies), so the compiler keeps five base registers and folds the
  // rest into the LDS instructions' immediate offsets instead of holding one
  // address register per (slot, row block, k-step).
  uint32_t lofs[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    lofs[q] = (lane & 31) * kStageBytes + (((2 * q + g) ^ swz_key<128>(lane & 31)) << 4);
  uint32_t lsc = S::kA + (lane & 31) * kDpr * 4;

  for (int64_t t = t_first; t < t_end; t += xs.nslots) {
    // ---- decode: virtual expert, then column tile (slow) and row tile (fast) ----
    int lo = 0, hi = V;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (static_cast<int64_t>(s_mt[mid]) * p.n_tiles <= t) lo = mid;
      else hi = mid;
    }
    const int v = lo;
    const int e = s_vmap[v];
    const bool dn = e >= E;                      // a part of the dense expert
    const int mtiles = s_mt[v + 1] - s_mt[v];
    const int64_t local = t - static_cast<int64_t>(s_mt[v]) * p.n_tiles;
    // a long segment's row tiles run in groups of kRowGroup: group, then
    // column tile, then row tile (the tiles an XCD runs at once cover
    // kRowGroup row tiles x a few column tiles, sharing both operands in its
    // L2); a segment of at most kRowGroup row tiles is one group
    const int grp = static_cast<int>(local / (kRowGroup * p.n_tiles));
    const int gm = min(kRowGroup, mtiles - kRowGroup * grp);
    const int idx = static_cast<int>(local - static_cast<int64_t>(grp) * kRowGroup * p.n_tiles);
    const int nt = idx / gm;
    const int mt = kRowGroup * grp + idx % gm;
    const int dlo = dn ? p.d_rows * (e - E) / kDenseParts : 0;   // first dense row of the part
    const int seg_lo = dn ? p.d_row0 + dlo : s_off[e];
    const int n_e = vrows(v);
    // A row of output row r: the gathered token row, the row itself, or for
    // the dense expert its own A rows
    auto a_row = [&](int r) {
      if (dn) return p.d_a_row0 + (r - p.d_row0);
      if (p.gather) {
        const int s = p.gather[r];
        return s < 0 ? 0 : s;  // padding row: loads any valid row, its output is zeroed
      }
      return r;
    };
    float* act_save = dn ? nullptr : p.act_save;
    int m_per = (n_e + mtiles - 1) / mtiles;
    m_per = (m_per + 31) & ~31;
    const int row0 = seg_lo + mt * m_per;
    const int nrows = min(m_per, n_e - mt * m_per);
    const int nrb = (nrows + 31) >> 5;
    const int cb0 = nt * 8 + 2 * wave;           // this wave's first column block
    const bool active = cb0 < p.ncb;             // uniform per wave

    // ---- per-lane sources (rows past the tile's end clamp to its last row) ----
    // source row (token row with gather) of A load i; byte offsets stay
    // below 2^31 for every layer shape (rows * row bytes)
    uint32_t a_off[kAIns];
#pragma unroll
    for (int i = 0; i < kAIns; ++i) {
      const int r = 8 * (wave + 4 * i) + (lane >> 3);
      const int src = a_row(row0 + min(r, nrows - 1));
      a_off[i] = static_cast<uint32_t>(src) * static_cast<uint32_t>(p.a_row_bytes) +
                 (((lane & 7) ^ swz_key<128>(r)) << 4);
    }
    if (p.gather && EPI == XEPI_SWIGLU)
      for (int r = tid; r < kRows; r += 256) s_src[r] = r < nrows && !dn ? p.gather[row0 + r] : 0;
    uint32_t asc_off[kAScPerWave > 0 ? kAScPerWave : 1];
    if constexpr (kSB > 0) {
#pragma unroll
      for (int q = 0; q < kAScPerWave; ++q) {
        const int j = min(wave + 4 * q, kAScIns - 1);  // covers rows [j * kScRows, +kScRows)
        const int r = min(j * kScRows + lane / kDpr, nrows - 1);
        const int src = a_row(row0 + r);
        asc_off[q] = static_cast<uint32_t>(src) * static_cast<uint32_t>(p.a_sc_row_bytes) + (lane % kDpr) * 4;
      }
    }
    const __amdgpu_buffer_rsrc_t a_rs = buf_rsrc(p.a, p.a_bytes);
    const __amdgpu_buffer_rsrc_t asc_rs = buf_rsrc(kSB > 0 ? p.a_sc : p.a, kSB > 0 ? p.a_sc_bytes : 0u);
    const int cbw = active ? cb0 : 0;
    const uint8_t* b_exp = dn ? p.d_b : p.b + static_cast<int64_t>(e) * p.b_exp_bytes;
    const uint8_t* b_src = b_exp + static_cast<int64_t>(cbw) * p.k_stages * O::kChunkW + lane * 16;
    const int64_t b_blk = static_cast<int64_t>(p.k_stages) * O::kChunkW;   // next column block
    const uint8_t* bsc_src = nullptr;
    int64_t bsc_blk = 0;
    if constexpr (OP != XOP_BF16) {
      const uint8_t* bsc_exp = dn ? p.d_b_sc : p.b_sc + static_cast<int64_t>(e) * p.b_sc_exp_bytes;
      bsc_src = bsc_exp + static_cast<int64_t>(cbw) * p.k_stages * O::kPackedScaleBytes +
                (OP == XOP_NVFP4 ? (lane & 31) * 4 : lane * kSub);
      bsc_blk = static_cast<int64_t>(p.k_stages) * O::kPackedScaleBytes;
    }

    const int KT = p.k_stages;

    // the weight ring: 4 pieces x 2 column blocks per stage (+ 2 scale words)
    u32x4_t bq[P][2][4];
    uint32_t bs[P][2];

    // One stage of loads is kPer(NV) operations per wave: 8 weight loads
    // (+2 MX scale words), NV activation row loads and kAScPerWave MX
    // scale loads of the rows, whatever the row count and whether the wave
    // has columns (rows past the tile's end re-read its last row, an idle
    // wave re-reads column block 0), so the vector-memory count of a stage
    // is a compile-time constant for both the explicit waits and the
    // compiler's own. issue_op(kt, slot, op) issues operation op of stage kt.
    auto issue_op = [&](int kt, auto slot_c, auto nv_c, auto op_c) {
      constexpr int SL = decltype(slot_c)::value;
      constexpr int NV = decltype(nv_c)::value;
      constexpr int OPN = decltype(op_c)::value;
      constexpr int kB = O::kBLoads;
      constexpr int kW = 2 * O::kPieces;
      if constexpr (OPN < kW) {
        constexpr int c = OPN / O::kPieces, q = OPN % O::kPieces;
        const uint8_t* bp = b_src + static_cast<int64_t>(kt) * O::kChunkW;
        bq[SL][c][q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(bp + c * b_blk + q * kPiece));
      } else if constexpr (OPN < kB) {
        constexpr int c = OPN - kW;
        const uint8_t* sp = bsc_src + static_cast<int64_t>(kt) * O::kPackedScaleBytes + c * bsc_blk;
        if constexpr (OP == XOP_FP8) bs[SL][c] = *reinterpret_cast<const uint16_t*>(sp);
        else bs[SL][c] = *reinterpret_cast<const uint32_t*>(sp);
      } else if constexpr (OPN < kB + NV) {
        constexpr int i = OPN - kB;
        uint8_t* st = smem + SL * S::kStage;
        lds_load16_buf(a_rs, a_off[i], static_cast<uint32_t>(kt) * kStageBytes, st + (wave + 4 * i) * 1024);
      } else {
        constexpr int q = OPN - kB - NV;
        uint8_t* st = smem + SL * S::kStage;
        lds_load4_buf(asc_rs, asc_off[q], static_cast<uint32_t>(kt) * kSB,
                      st + S::kA + min(wave + 4 * q, kAScIns - 1) * 256);
      }
    };
    // a whole stage, activation operations first (the order the steps use)
    auto issue = [&](int kt, auto slot_c, auto nv_c) {
      constexpr int NV = decltype(nv_c)::value;
      constexpr int kB = O::kBLoads;
      constexpr int kPer = kB + NV + kAScPerWave;
      static_for<kPer>([&](auto op_c) {
        issue_op(kt, slot_c, nv_c, std::integral_constant<int, (decltype(op_c)::value + kB) % kPer>{});
      });
    };

    f32x16_t acc[MAXNV][2];
#pragma unroll
    for (int i = 0; i < MAXNV; ++i) {
      acc[i][0] = f32x16_t{};
      acc[i][1] = f32x16_t{};
    }

    // MFMAs of one stage for the first NV row blocks. The (k-step, row
    // block) sequence is walked with the activation operands (and their MX
    // scale words) read from LDS one or two steps ahead into a small
    // register ring, so LDS latency hides behind the matrix instructions of
    // the previous steps.
    // The weight loads of the stage P-1 ahead (kt_next, into register slot
    // NSL) are spread over the steps, so the memory pipeline works while the
    // matrix cores do. (The direct-to-LDS activation loads of that stage are
    // issued right after the barrier instead: spread among the LDS operand
    // reads they gave run-to-run differences on gfx950.)
    auto compute = [&](auto slot_c, auto nv_c, int kt_next, auto nslot_c) {
      constexpr int SL = decltype(slot_c)::value;
      constexpr int NV = decltype(nv_c)::value;
      constexpr int NSTEP = kSub * NV;
      constexpr int kB = O::kBLoads;  // weight loads per stage
      // operand ring depth: reads D - 1 steps ahead (an E4M3 step's two
      // 64-cycle MFMAs cover one LDS read; bf16 and E2M1 steps take 32 cycles
      // per MFMA and read two steps ahead)
      constexpr int D = OP == XOP_FP8 ? 2 : 3;
      // this slot's per-lane operand offsets; the row block's offset (32
      // rows = 4 KB) and the scale word's are immediates of the LDS reads
      uint32_t vo[4], vs;
#pragma unroll
      for (int q = 0; q < 4; ++q) vo[q] = lofs[q] + SL * S::kStage;
      vs = lsc + SL * S::kStage;
      using AFrag = std::conditional_t<O::kBf16A, bf16x8_t, i32x8_t>;
      AFrag afr[D];
      uint32_t asw[D];
      bf16x8_t bcv[2];   // NVFP4: this k-step's weight operands converted to bf16
      auto fetch = [&](auto st_c) {
        constexpr int ST = decltype(st_c)::value;
        constexpr int s = ST / NV, i = ST % NV, buf = ST % D;
        constexpr int ri = 32 * kStageBytes * i;
        if constexpr (O::kBf16A) {
          afr[buf] = *reinterpret_cast<const bf16x8_t*>(smem + vo[s] + ri);
        } else {
          if constexpr (OP == XOP_FP8) {
            const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(smem + vo[2 * s] + ri);
            const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(smem + vo[2 * s + 1] + ri);
            afr[buf] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          } else {
            const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(smem + vo[s] + ri);
            afr[buf] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], 0, 0, 0, 0};
          }
          // word (2 s + g) / 4 = s / 2 of the row's scale dwords
          asw[buf] = *reinterpret_cast<const uint32_t*>(smem + vs + 4 * (32 * kDpr * i + (s >> 1)));
        }
      };
      static_for<(NSTEP < D - 1 ? NSTEP : D - 1)>([&](auto st_c) { fetch(st_c); });
      static_for<NSTEP>([&](auto st_c) {
        constexpr int ST = decltype(st_c)::value;
        constexpr int s = ST / NV, i = ST % NV, buf = ST % D;
        if constexpr (ST + D - 1 < NSTEP) fetch(std::integral_constant<int, ST + D - 1>{});
        static_for<(ST + 1) * kB / NSTEP - ST * kB / NSTEP>([&](auto o_c) {
          issue_op(kt_next, nslot_c, nv_c, std::integral_constant<int, ST * kB / NSTEP + decltype(o_c)::value>{});
        });
        // keep the reads of step ST+D-1 and the loads ahead of the MFMAs of
        // step ST (the scheduler would otherwise sink them next to their use)
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (OP == XOP_BF16) {
          const bf16x8_t b0 = __builtin_bit_cast(bf16x8_t, bq[SL][0][s]);
          const bf16x8_t b1 = __builtin_bit_cast(bf16x8_t, bq[SL][1][s]);
          if constexpr (kRowsInLanes) {
            acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0, afr[buf], acc[i][0], 0, 0, 0);
            acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1, afr[buf], acc[i][1], 0, 0, 0);
          } else {
            acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[buf], b0, acc[i][0], 0, 0, 0);
            acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[buf], b1, acc[i][1], 0, 0, 0);
          }
        } else if constexpr (OP == XOP_NVFP4) {
          // the lane's 8 codes of k-step s (dword s of its 16-byte load) times
          // their E4M3 block scale (byte s of its scale word): E2M1 -> fp32
          // with unit scale (exact), one fp32 product per value (exact: at
          // most 6 significant bits), the high halves packed as bf16 (exact);
          // converted once per k-step for all row blocks
          if constexpr (i == 0) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const uint32_t w = bq[SL][c][0][s];
              const float sc = e4m3_value((bs[SL][c] >> (8 * s)) & 0xFFu);
              uint32_t pk[4];
              static_for<4>([&](auto b_c) {
                const f32x2_t f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.f, decltype(b_c)::value);
                pk[decltype(b_c)::value] = __builtin_amdgcn_perm(__float_as_uint(f[1] * sc),
                                                                 __float_as_uint(f[0] * sc), 0x07060302u);
              });
              bcv[c] = __builtin_bit_cast(bf16x8_t, u32x4_t{pk[0], pk[1], pk[2], pk[3]});
            }
          }
          if constexpr (kRowsInLanes) {
            acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bcv[0], afr[buf], acc[i][0], 0, 0, 0);
            acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bcv[1], afr[buf], acc[i][1], 0, 0, 0);
          } else {
            acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[buf], bcv[0], acc[i][0], 0, 0, 0);
            acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[buf], bcv[1], acc[i][1], 0, 0, 0);
          }
        } else {
          i32x8_t b0, b1;
          if constexpr (OP == XOP_FP8) {
            const u32x4_t l0 = bq[SL][0][2 * s], h0 = bq[SL][0][2 * s + 1];
            const u32x4_t l1 = bq[SL][1][2 * s], h1 = bq[SL][1][2 * s + 1];
            b0 = i32x8_t{(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3], (int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3]};
            b1 = i32x8_t{(int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
          } else {
            const u32x4_t l0 = bq[SL][0][s], l1 = bq[SL][1][s];
            b0 = i32x8_t{(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3], 0, 0, 0, 0};
            b1 = i32x8_t{(int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3], 0, 0, 0, 0};
          }
          const int bs0 = static_cast<int>((bs[SL][0] >> (8 * s)) & 0xFFu);
          const int bs1 = static_cast<int>((bs[SL][1] >> (8 * s)) & 0xFFu);
          const int as = static_cast<int>((asw[buf] >> (8 * ((2 * s + g) & 3))) & 0xFFu);
          constexpr int fmt = OP == XOP_FP8 ? 0 : 4;
          if constexpr (kRowsInLanes) {
            acc[i][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b0, afr[buf], acc[i][0], fmt, fmt, 0, bs0, 0, as);
            acc[i][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b1, afr[buf], acc[i][1], fmt, fmt, 0, bs1, 0, as);
          } else {
            acc[i][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(afr[buf], b0, acc[i][0], fmt, fmt, 0, as, 0, bs0);
            acc[i][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(afr[buf], b1, acc[i][1], fmt, fmt, 0, as, 0, bs1);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    };

    // ---- main loop: stage kt waits for its loads, frees slot (kt-1)%P by
    // the barrier, then computes while issuing stage kt+P-1 into that slot.
    // Every step issues its stage's activation loads first, then the weight
    // loads, and its wait also covers the activation loads of the next stage
    // (only that stage's weight loads stay in flight): the direct-to-LDS
    // loads are complete a whole step before any wave reads them. (Waiting
    // for them only at the step that reads them let, on gfx950, a few rows
    // of a wave's last activation load per stage be read stale now and then:
    // run-to-run differences in ~1% of the rows of the bf16 fc2 at 4096
    // tokens x 256 experts, none with the earlier wait.)
    // Every wave computes (a wave without columns works on duplicate data
    // it never stores) and every iteration issues exactly one stage (past
    // the end it re-issues the last stage, whose data nobody reads), so the
    // steady-state loop has a single path and the wait count is a constant.
    // Whole groups of P stages run unconditionally; the last KT % P stages
    // follow in a short tail. ----
    auto run = [&](auto nv_c) {
      constexpr int NV = decltype(nv_c)::value;
      constexpr int kPer = NV + kAScPerWave + O::kBLoads;  // loads per stage
      static_assert((P - 2) * kPer <= 62, "vmcnt range");
      // loads still allowed in flight at a step's wait: the weight loads of
      // the stages after the next (none with a two-stage ring)
      constexpr int kWait = P > 2 ? (P - 2) * kPer - NV - kAScPerWave : 0;
      static_for<P - 1>([&](auto s_c) {
        issue(min(static_cast<int>(decltype(s_c)::value), KT - 1), s_c, nv_c);
      });
      auto step = [&](int kt, auto j_c) {
        constexpr int J = decltype(j_c)::value;
        constexpr int kB = O::kBLoads;
        using NSL = std::integral_constant<int, (J + P - 1) % P>;
        const int kt_next = min(kt + P - 1, KT - 1);
        asm volatile("" : "+v"(lofs[0]), "+v"(lofs[1]), "+v"(lofs[2]), "+v"(lofs[3]), "+v"(lsc));
        wait_vmcnt<kWait>();
        lds_barrier();
        static_for<NV + kAScPerWave>([&](auto o_c) {
          issue_op(kt_next, NSL{}, nv_c, std::integral_constant<int, kB + decltype(o_c)::value>{});
        });
        __builtin_amdgcn_sched_barrier(0);  // the weight loads stay behind them
        compute(j_c, nv_c, kt_next, NSL{});
      };
      int k0 = 0;
      for (; k0 + P <= KT; k0 += P) static_for<P>([&](auto j_c) { step(k0 + decltype(j_c)::value, j_c); });
      static_for<P - 1>([&](auto j_c) {
        if (k0 + decltype(j_c)::value < KT) step(k0 + decltype(j_c)::value, j_c);
      });
    };
    switch (min(nrb, MAXNV)) {
#define MOE_NV(N) case N: if constexpr (N <= MAXNV) run(std::integral_constant<int, N>{}); break;
      MOE_NV(1) MOE_NV(2) MOE_NV(3) MOE_NV(4) MOE_NV(5) MOE_NV(6) MOE_NV(7) MOE_NV(8)
#undef MOE_NV
      default: break;
    }
    // every wave is done with the LDS ring, and every direct-to-LDS load
    // (the tail re-issues the last stage) has landed before the epilogue
    // reuses that LDS: the workgroup barrier by itself need not wait for
    // them, so the wait is explicit
    wait_vmcnt<0>();
    __syncthreads();

    if constexpr (kRowsInLanes) {
      // ---- plain epilogue from registers: in a 32x32 block lane l holds
      // row l % 32 and, in registers 4k..4k+3, columns 8k + 4g + 0..3 (g =
      // l / 32). One permlane32 swap per dword pair of the blocks k and k+2
      // gives lane l < 32 columns [8k', 8k' + 8) and lane l + 32 columns
      // [16 + 8k', 16 + 8k' + 8) (k' = k); so lane l writes columns [0, 16)
      // and lane l + 32 columns [16, 32) of its row, 32 contiguous bytes ----
      const float gs = OP == XOP_NVFP4 ? p.a_g * p.w_g[e] : 1.f;
      if (active) {
#pragma unroll
        for (int i = 0; i < MAXNV; ++i) {
          const int r = 32 * i + (lane & 31);
          if (i < nrb) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const f32x16_t& a = acc[i][c];
              uint32_t w[8];
#pragma unroll
              for (int k = 0; k < 2; ++k) {
                // blocks k (columns 8k + 4g ..) and k + 2 (16 + 8k + 4g ..)
                const uint32_t x0 = pack_bf16x2(a[4 * k] * gs, a[4 * k + 1] * gs);
                const uint32_t x1 = pack_bf16x2(a[4 * k + 2] * gs, a[4 * k + 3] * gs);
                const uint32_t y0 = pack_bf16x2(a[4 * k + 8] * gs, a[4 * k + 9] * gs);
                const uint32_t y1 = pack_bf16x2(a[4 * k + 10] * gs, a[4 * k + 11] * gs);
                const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
                w[4 * k + 0] = s0[0];
                w[4 * k + 1] = s1[0];
                w[4 * k + 2] = s0[1];
                w[4 * k + 3] = s1[1];
              }
              if (r < nrows) {
                const int col = nt * kTileCols + 64 * wave + 32 * c + 16 * g;
                u32x4_t* o = reinterpret_cast<u32x4_t*>(p.out + static_cast<int64_t>(row0 + r) * p.out_row_bytes +
                                                        static_cast<int64_t>(col) * 2);
                o[0] = u32x4_t{w[0], w[1], w[2], w[3]};
                o[1] = u32x4_t{w[4], w[5], w[6], w[7]};
              }
            }
          }
        }
      }
      continue;
    }

    // ---- epilogue in passes of up to 128 rows through an fp32 LDS tile ----
    // C layout of a 32x32 MFMA: lane l, element r -> row 8*(r/4) + 4*(l/32) + r%4, column l%32
    float* cs = reinterpret_cast<float*>(smem);
    // NVFP4: the accumulators hold sums of (code * scale) products; the
    // activation and the expert's weight tensor scales multiply them here
    const float gs = OP == XOP_NVFP4 ? p.a_g * p.w_g[e] : 1.f;
    constexpr int kPassRB = kPassRows / 32 < MAXNV ? kPassRows / 32 : MAXNV;
    for (int pass = 0; pass * kPassRB < nrb; ++pass) {
      const int prow0 = pass * kPassRB * 32;
      const int prows = min(kPassRB * 32, nrows - prow0);
      if (active) {
#pragma unroll
        for (int i = 0; i < MAXNV; ++i) {
          if (i / kPassRB == pass && i < nrb) {
            if (EPI == XEPI_SWIGLU && OUTF != MOE_BF16 && !act_save) {
              // MX-encoded h: a wave holds the gate block and the up block
              // of the same 32 h columns in one layout, so h = silu(g) * u
              // is formed in registers and only h goes through LDS (columns
              // [0, 128)) to the block encoder
              const int hcol = 32 * wave + (lane & 31);
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int row = (i - pass * kPassRB) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                cs[row * kCs + hcol] = silu_mul(acc[i][0][r] * gs, acc[i][1][r] * gs);
              }
            } else {
              // gate | up (SwiGLU with the fp32 save) or the plain tile
#pragma unroll
              for (int c = 0; c < 2; ++c) {
                const int col = EPI == XEPI_SWIGLU ? 128 * c + 32 * wave + (lane & 31)
                                                   : 64 * wave + 32 * c + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                  const int row = (i - pass * kPassRB) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                  cs[row * kCs + col] = OP == XOP_NVFP4 ? acc[i][c][r] * gs : acc[i][c][r];
                }
              }
            }
          }
        }
      }
      __syncthreads();
      if constexpr (EPI == XEPI_SWIGLU) {
        const int F = p.half;
        const int hc0 = nt * 128;                        // first h column of the tile
        const int width = min(128, F - hc0);
        if constexpr (OUTF == MOE_BF16) {
          for (int i = tid; i < prows * (width / 8); i += 256) {
            const int row = i / (width / 8), c0 = (i % (width / 8)) * 8;
            const bool zero = p.gather && s_src[prow0 + row] < 0;
            const float* gp = cs + row * kCs + c0;
            float h[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) h[q] = zero ? 0.f : silu_mul(gp[q], gp[128 + q]);
            const int64_t grow = row0 + prow0 + row;
            *reinterpret_cast<u32x4_t*>(p.out + grow * p.out_row_bytes + (hc0 + c0) * 2) =
                u32x4_t{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]), pack_bf16x2(h[4], h[5]),
                        pack_bf16x2(h[6], h[7])};
            if (act_save) {
              float* ar = act_save + grow * (2ll * F) + hc0 + c0;
              store8_f32(ar, gp);
              store8_f32(ar + F, gp + 128);
            }
          }
        } else if constexpr (OUTF == MOE_NVFP4_E2M1) {
          // h (formed in registers above, columns [0, 128) of the tile) in
          // blocks of 16 -> NVFP4 with the tensor scale of h; stored as the
          // operand values code * scale (bf16, exact) that fc2 consumes
          const int nblk = width / 16;
          const float d6 = 6.f * p.out_g;
          for (int i = tid; i < prows * nblk; i += 256) {
            const int row = i / nblk, blk = i % nblk;
            const bool zero = p.gather && s_src[prow0 + row] < 0;
            const float* gp = cs + row * kCs + blk * 16;
            float v[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) v[q] = zero ? 0.f : gp[q];
            uint32_t cw[2], vw[8];
            nvfp4_encode_block(v, p.out_g, d6, cw, vw);
            const int64_t grow = row0 + prow0 + row;
            u32x4_t* o = reinterpret_cast<u32x4_t*>(p.out + grow * p.out_row_bytes + (hc0 + blk * 16) * 2);
            o[0] = u32x4_t{vw[0], vw[1], vw[2], vw[3]};
            o[1] = u32x4_t{vw[4], vw[5], vw[6], vw[7]};
          }
        } else {
          constexpr bool fp4 = OUTF == MOE_MXFP4_E2M1;
          const int nblk = width / 32;
          for (int i = tid; i < prows * nblk; i += 256) {
            const int row = i / nblk, blk = i % nblk;
            const bool zero = p.gather && s_src[prow0 + row] < 0;
            const float* gp = cs + row * kCs + blk * 32;
            float v[32];
            if (!act_save) {
#pragma unroll
              for (int q = 0; q < 32; ++q) v[q] = zero ? 0.f : gp[q];
            } else {
#pragma unroll
              for (int q = 0; q < 32; ++q) v[q] = zero ? 0.f : silu_mul(gp[q], gp[128 + q]);
            }
            uint32_t words[8];
            const uint32_t sb = mx_encode_block<fp4>(v, words);
            const int64_t grow = row0 + prow0 + row;
            const int gblk = hc0 / 32 + blk;
            if (fp4) {
              *reinterpret_cast<u32x4_t*>(p.out + grow * p.out_row_bytes + gblk * 16) =
                  u32x4_t{words[0], words[1], words[2], words[3]};
            } else {
              u32x4_t* o = reinterpret_cast<u32x4_t*>(p.out + grow * p.out_row_bytes + gblk * 32);
              o[0] = u32x4_t{words[0], words[1], words[2], words[3]};
              o[1] = u32x4_t{words[4], words[5], words[6], words[7]};
            }
            p.out_sc[grow * p.out_sc_row_bytes + gblk] = static_cast<uint8_t>(sb);
            if (act_save) {
              float* ar = act_save + grow * (2ll * F) + hc0 + blk * 32;
#pragma unroll
              for (int q = 0; q < 32; q += 8) {
                store8_f32(ar + q, gp + q);
                store8_f32(ar + F + q, gp + 128 + q);
              }
            }
          }
        }
      } else if constexpr (EPI == XEPI_PLAIN) {
        const int c_first = nt * kTileCols;
        const int width = min(kTileCols, p.ncb * 32 - c_first);
        for (int i = tid; i < prows * (width / 8); i += 256) {
          const int row = i / (width / 8), c0 = (i % (width / 8)) * 8;
          const float* v = cs + row * kCs + c0;
          *reinterpret_cast<u32x4_t*>(p.out + static_cast<int64_t>(row0 + prow0 + row) * p.out_row_bytes +
                                      static_cast<int64_t>(c_first + c0) * 2) =
              u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                      pack_bf16x2(v[6], v[7])};
        }
      } else {
        // dSwiGLU: the tile holds dH for F columns [256 nt, +width); with the
        // saved fc1 output (g | u): dgate = dH * u * sig(g) * (1 + g * (1 - sig(g))),
        // dup = dH * silu(g)
        const int F = p.half;
        const int64_t a2 = 2ll * F;
        const int c_first = nt * kTileCols;
        const int width = min(kTileCols, F - c_first);
        if constexpr (OUTF == MOE_BF16) {
          for (int i = tid; i < prows * (width / 8); i += 256) {
            const int row = i / (width / 8), c0 = (i % (width / 8)) * 8;
            const int col = c_first + c0;
            const int64_t grow = row0 + prow0 + row;
            float gv[8], uv[8], dg[8], du[8];
            load8_f32(p.a_saved + grow * a2 + col, gv);
            load8_f32(p.a_saved + grow * a2 + F + col, uv);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const float dh = cs[row * kCs + c0 + q];
              const float sg = sigmoidf_(gv[q]);
              dg[q] = dh * uv[q] * sg * (1.f + gv[q] * (1.f - sg));
              du[q] = dh * (gv[q] * sg);
            }
            uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + grow * a2;
            *reinterpret_cast<u32x4_t*>(o + col) =
                u32x4_t{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]), pack_bf16x2(dg[4], dg[5]),
                        pack_bf16x2(dg[6], dg[7])};
            *reinterpret_cast<u32x4_t*>(o + F + col) =
                u32x4_t{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]), pack_bf16x2(du[4], du[5]),
                        pack_bf16x2(du[6], du[7])};
            if (p.da_f32) {
              store8_f32(p.da_f32 + grow * a2 + col, dg);
              store8_f32(p.da_f32 + grow * a2 + F + col, du);
            }
          }
        } else {
          constexpr bool fp4 = OUTF == MOE_MXFP4_E2M1;
          constexpr int kBlkBytes = fp4 ? 16 : 32;
          const int nblk = width / 32;
          // one item per (row, 32-column block, half): the gate half's or
          // the up half's 32 gradients are formed, encoded and stored on
          // their own (both at once hold 64 values in registers)
          for (int i = tid; i < prows * nblk * 2; i += 256) {
            const int half = i & 1, item = i >> 1;
            const int row = item / nblk, blk = item % nblk;
            const int col = c_first + blk * 32;
            const int64_t grow = row0 + prow0 + row;
            float v[32];
#pragma unroll
            for (int w8 = 0; w8 < 4; ++w8) {
              float gv[8], uv[8];
              load8_f32(p.a_saved + grow * a2 + col + w8 * 8, gv);
              load8_f32(p.a_saved + grow * a2 + F + col + w8 * 8, uv);
#pragma unroll
              for (int q = 0; q < 8; ++q) {
                const float dh = cs[row * kCs + blk * 32 + w8 * 8 + q];
                const float sg = sigmoidf_(gv[q]);
                v[w8 * 8 + q] = half ? dh * (gv[q] * sg) : dh * uv[q] * sg * (1.f + gv[q] * (1.f - sg));
              }
            }
            uint32_t words[8];
            const int c = half ? F + col : col;
            const uint32_t sb = mx_encode_block<fp4>(v, words);
            u32x4_t* o = reinterpret_cast<u32x4_t*>(p.out + grow * p.out_row_bytes + (c / 32) * kBlkBytes);
            o[0] = u32x4_t{words[0], words[1], words[2], words[3]};
            if (!fp4) o[1] = u32x4_t{words[4], words[5], words[6], words[7]};
            p.out_sc[grow * p.out_sc_row_bytes + c / 32] = static_cast<uint8_t>(sb);
            if (p.da_f32) {
              float* ob = p.da_f32 + grow * a2 + c;
#pragma unroll
              for (int w8 = 0; w8 < 4; ++w8) store8_f32(ob + w8 * 8, v + w8 * 8);
            }
          }
        }
      }
      __syncthreads();  // the LDS tile is rewritten by the next pass / tile
    }
  }
}

// ---- weight packing ---------------------------------------------------------
// packed[e][cb][s][q][lane][16 B] = row R(cb, lane % 32) of expert e, bytes
// [128 s + 32 q + 16 (lane / 32), +16), where R is 32 cb + lane % 32, or with
// gate/up pairing (half = F > 0) gate row 32 (cb / 2) + lane % 32 for even cb
// and up row F + 32 (cb / 2) + lane % 32 for odd cb.
// packed scales [e][cb][s][lane][j] = scale of that row's MX block
// (stage-local) 2 j + lane / 32, j < kSub.
__device__ __forceinline__ int packed_row(int cb, int lane, int half) {
  if (half > 0) return ((cb & 1) ? half : 0) + 32 * (cb >> 1) + (lane & 31);
  return 32 * cb + (lane & 31);
}

__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t* __restrict__ w, int64_t E,
                                                         int N, int64_t kbytes, int half,
                                                         uint8_t* __restrict__ out) {
  const int ncb = N / 32;
  const int64_t S = kbytes / kStageBytes;
  const int64_t total = E * ncb * S * 4 * 64;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < total; i += 256ll * gridDim.x) {
    const int lane = static_cast<int>(i & 63);
    const int q = static_cast<int>((i >> 6) & 3);
    const int64_t rest = i >> 8;
    const int64_t s = rest % S;
    const int64_t cbe = rest / S;
    const int cb = static_cast<int>(cbe % ncb);
    const int64_t e = cbe / ncb;
    const int64_t row = e * N + packed_row(cb, lane, half);
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(w + row * kbytes + s * kStageBytes + 32 * q + 16 * (lane >> 5));
    *reinterpret_cast<u32x4_t*>(out + i * 16) = v;
  }
}

__global__ __launch_bounds__(256) void pack_scales_kernel(const uint8_t* __restrict__ sc, int64_t E,
                                                          int N, int64_t kblocks, int sub, int half,
                                                          uint8_t* __restrict__ out) {
  const int ncb = N / 32;
  const int64_t blocks_per_stage = 2 * sub;  // MX blocks of 32 per stage
  const int64_t S = kblocks / blocks_per_stage;
  const int64_t total = E * ncb * S * 64 * sub;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < total; i += 256ll * gridDim.x) {
    const int j = static_cast<int>(i % sub);
    const int64_t li = i / sub;
    const int lane = static_cast<int>(li & 63);
    const int64_t rest = li >> 6;
    const int64_t s = rest % S;
    const int64_t cbe = rest / S;
    const int cb = static_cast<int>(cbe % ncb);
    const int64_t e = cbe / ncb;
    const int64_t row = e * N + packed_row(cb, lane, half);
    out[i] = sc[row * kblocks + s * blocks_per_stage + 2 * j + (lane >> 5)];
  }
}

// NVFP4 weights for the bf16 k-steps (16 values): packed[e][cb][s][lane]
// 16 bytes = for k-step ks < 4 the 4 code bytes of row R(cb, lane) at byte
// 32 s + 8 ks + 4 (lane / 32) (the lane's 8 values of the k-step); scales
// [e][cb][s][r < 32] 4 bytes = for ks < 4 the E4M3 scale of row R(cb, r)'s
// block 4 s + ks (one block of 16 per k-step, read by both lane halves):
// as many bytes as the unpacked scales.
__global__ __launch_bounds__(256) void pack_nvfp4_codes_kernel(const uint8_t* __restrict__ w, int64_t E,
                                                               int N, int64_t kbytes, int half,
                                                               uint8_t* __restrict__ out) {
  const int ncb = N / 32;
  const int64_t S = kbytes / 32;     // 64-value stages
  const int64_t total = E * ncb * S * 64;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < total; i += 256ll * gridDim.x) {
    const int lane = static_cast<int>(i & 63);
    const int64_t rest = i >> 6;
    const int64_t s = rest % S;
    const int64_t cbe = rest / S;
    const int cb = static_cast<int>(cbe % ncb);
    const int64_t e = cbe / ncb;
    const uint8_t* row = w + (e * N + packed_row(cb, lane, half)) * kbytes + 32 * s + 4 * (lane >> 5);
    u32x4_t v;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) v[ks] = *reinterpret_cast<const uint32_t*>(row + 8 * ks);
    *reinterpret_cast<u32x4_t*>(out + i * 16) = v;
  }
}

__global__ __launch_bounds__(256) void pack_nvfp4_scales_kernel(const uint8_t* __restrict__ sc, int64_t E,
                                                                int N, int64_t kblocks, int half,
                                                                uint8_t* __restrict__ out) {
  const int ncb = N / 32;
  const int64_t S = kblocks / 4;
  const int64_t total = E * ncb * S * 32;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < total; i += 256ll * gridDim.x) {
    const int r = static_cast<int>(i & 31);
    const int64_t rest = i >> 5;
    const int64_t s = rest % S;
    const int64_t cbe = rest / S;
    const int cb = static_cast<int>(cbe % ncb);
    const int64_t e = cbe / ncb;
    const uint8_t* src = sc + (e * N + packed_row(cb, r, half)) * kblocks + 4 * s;
    reinterpret_cast<uint32_t*>(out)[i] = static_cast<uint32_t>(src[0]) | (static_cast<uint32_t>(src[1]) << 8) |
                                          (static_cast<uint32_t>(src[2]) << 16) |
                                          (static_cast<uint32_t>(src[3]) << 24);
  }
}

}  // namespace

int xop_of(int fmt) {
  return fmt == MOE_BF16 ? XOP_BF16
                         : (fmt == MOE_MXFP8_E4M3 ? XOP_FP8 : (fmt == MOE_NVFP4_E2M1 ? XOP_NVFP4 : XOP_FP4));
}

// Launch of one grouped expert GEMM with packed weights (expert_gemm.h).
int expert_gemm(int kind, const void* a, const uint8_t* a_scales, int fmt, const int32_t* gather,
                const void* wp, const uint8_t* wp_scales, const int32_t* offsets, int E, int N,
                int K, int64_t rows, int half, void* out, uint8_t* out_scales, float* act_save,
                const float* a_saved, float* da_f32, hipStream_t stream,
                const DenseExpert* dense, const NvScales* nv) {
  // bits of an activation element and of a stored weight element (the
  // NVFP4 activation operand arrives as bf16 values code * scale)
  const bool nvfp4 = fmt == MOE_NVFP4_E2M1;
  const int bits = fmt == MOE_BF16 || nvfp4 ? 16 : (fmt == MOE_MXFP8_E4M3 ? 8 : 4);
  const int wbits = fmt == MOE_BF16 ? 16 : (fmt == MOE_MXFP8_E4M3 ? 8 : 4);
  MOE_REQUIRE(!nvfp4 || (nv && kind != 2 && !(dense && dense->rows > 0)), MOE_ERR_UNSUPPORTED,
              "grouped expert GEMM: NVFP4 runs fc1 / fc2 of routed experts only, with its scales");
  // activation row offsets are 32-bit inside the kernel; a gathered source
  // has at most `rows` rows as well
  const int64_t a_rows =
      dense && dense->rows > 0 ? std::max<int64_t>(rows, dense->a_row0 + int64_t{dense->rows}) : rows;
  MOE_REQUIRE(a_rows * (static_cast<int64_t>(K) * bits / 8) < (int64_t{1} << 32), MOE_ERR_UNSUPPORTED,
              "grouped expert GEMM: activation matrix of 4 GiB or more");
  MOE_REQUIRE(E + (dense && dense->rows > 0 ? kDenseParts : 0) <= kMaxVirt && E <= 32767,
              MOE_ERR_INVALID_ARG, "grouped expert GEMM: too many experts");
  XArgs x{};
  x.a = static_cast<const uint8_t*>(a);
  x.a_row_bytes = static_cast<int64_t>(K) * bits / 8;
  x.a_sc = a_scales;
  x.a_sc_row_bytes = K / 32;
  x.a_bytes = static_cast<uint32_t>(a_rows * x.a_row_bytes);
  x.a_sc_bytes = static_cast<uint32_t>(a_rows * (K / 32));
  x.gather = gather;
  x.b = static_cast<const uint8_t*>(wp);
  x.b_exp_bytes = static_cast<int64_t>(N) * K * wbits / 8;
  x.b_sc = wp_scales;
  x.b_sc_exp_bytes = static_cast<int64_t>(N) * (K / (nvfp4 ? 16 : 32));
  x.ncb = N / 32;
  x.n_tiles = kind == 0 ? (N / 2 + 127) / 128 : (N + kTileCols - 1) / kTileCols;
  x.k_stages = static_cast<int>(x.a_row_bytes / kStageBytes);
  x.offsets = offsets;
  x.E = E;
  x.rows = rows;
  x.half = half;
  x.out = static_cast<uint8_t*>(out);
  x.out_sc = out_scales;
  x.act_save = act_save;
  x.a_saved = a_saved;
  x.da_f32 = da_f32;
  if (nvfp4) {
    x.a_g = nv->a_g;
    x.w_g = nv->w_g;
    x.out_g = nv->out_g;
  }
  if (dense && dense->rows > 0) {
    x.d_b = static_cast<const uint8_t*>(dense->w);
    x.d_b_sc = dense->w_scales;
    x.d_rows = dense->rows;
    x.d_row0 = dense->row0;
    x.d_a_row0 = dense->a_row0;
  }
  const int outw = kind == 0 ? half : (kind == 1 ? N : 2 * half);  // output row elements
  const bool mx_out = kind != 1 && (fmt == MOE_MXFP8_E4M3 || fmt == MOE_MXFP4_E2M1);
  x.out_row_bytes = mx_out ? static_cast<int64_t>(outw) * bits / 8 : static_cast<int64_t>(outw) * 2;
  x.out_sc_row_bytes = outw / 32;
  const dim3 block(256);
  auto launch = [&](auto mn_c, auto pp_c, auto oc_c) {
    constexpr int MN = decltype(mn_c)::value, PP = decltype(pp_c)::value;
    constexpr int OC = decltype(oc_c)::value;
    const dim3 grid(kNumCu * OC);
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, block, 0, stream, x); };
    switch (kind * 4 + xop_of(fmt)) {
      case 0: go(expert_gemm_kernel<MN, PP, OC, XOP_BF16, XEPI_SWIGLU, MOE_BF16>); break;
      case 1: go(expert_gemm_kernel<MN, PP, OC, XOP_FP8, XEPI_SWIGLU, MOE_MXFP8_E4M3>); break;
      case 2: go(expert_gemm_kernel<MN, PP, OC, XOP_FP4, XEPI_SWIGLU, MOE_MXFP4_E2M1>); break;
      case 3: go(expert_gemm_kernel<MN, PP, OC, XOP_NVFP4, XEPI_SWIGLU, MOE_NVFP4_E2M1>); break;
      case 4: go(expert_gemm_kernel<MN, PP, OC, XOP_BF16, XEPI_PLAIN, MOE_BF16>); break;
      case 5: go(expert_gemm_kernel<MN, PP, OC, XOP_FP8, XEPI_PLAIN, MOE_BF16>); break;
      case 6: go(expert_gemm_kernel<MN, PP, OC, XOP_FP4, XEPI_PLAIN, MOE_BF16>); break;
      case 7: go(expert_gemm_kernel<MN, PP, OC, XOP_NVFP4, XEPI_PLAIN, MOE_BF16>); break;
      case 8: go(expert_gemm_kernel<MN, PP, OC, XOP_BF16, XEPI_DSWIGLU, MOE_BF16>); break;
      case 9: go(expert_gemm_kernel<MN, PP, OC, XOP_FP8, XEPI_DSWIGLU, MOE_MXFP8_E4M3>); break;
      default: go(expert_gemm_kernel<MN, PP, OC, XOP_FP4, XEPI_DSWIGLU, MOE_MXFP4_E2M1>); break;
    }
  };
  // decode batches (a few rows per expert on average): 64-row tiles and a
  // 6-deep ring keep more weight bytes in flight per wave
  using I = std::integral_constant<int, 1>;
  if (kind != 2 && rows <= 8ll * E)
    launch(std::integral_constant<int, 2>{}, std::integral_constant<int, 6>{}, I{});
  else
    launch(std::integral_constant<int, 8>{}, std::integral_constant<int, 3>{}, I{});
  return check_launch("grouped expert GEMM");
}

}  // namespace moe

using namespace moe;

extern "C" int moe_pack_weights(const void* w, const uint8_t* w_scales, int fmt, int E, int N,
                                int K, int half, void* out, uint8_t* out_scales,
                                hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(E >= 1 && N > 0 && K > 0, MOE_ERR_INVALID_ARG, "moe_pack_weights: need E, N, K > 0");
  MOE_REQUIRE(fmt == MOE_BF16 || fmt == MOE_MXFP8_E4M3 || fmt == MOE_MXFP4_E2M1 ||
                  fmt == MOE_NVFP4_E2M1,
              MOE_ERR_UNSUPPORTED, "moe_pack_weights: fmt must be MOE_BF16, an MX format or NVFP4");
  if (fmt == MOE_NVFP4_E2M1) {
    MOE_REQUIRE(N % 64 == 0 && K % 64 == 0, MOE_ERR_INVALID_ARG,
                "moe_pack_weights: NVFP4 needs N % 64 == 0 and K % 64 == 0");
    MOE_REQUIRE(half == 0 || (half > 0 && N == 2 * half && half % 32 == 0), MOE_ERR_INVALID_ARG,
                "moe_pack_weights: gate/up pairing needs N == 2 * half and half % 32 == 0");
    MOE_REQUIRE(w && out && w_scales && out_scales, MOE_ERR_INVALID_ARG, "moe_pack_weights: null pointer");
    MOE_REQUIRE(aligned16(w) && aligned16(out) && (reinterpret_cast<uintptr_t>(out_scales) & 3u) == 0,
                MOE_ERR_ALIGNMENT, "moe_pack_weights: w and out must be 16-byte, out_scales 4-byte aligned");
    const int64_t items = static_cast<int64_t>(E) * (N / 32) * (K / 64) * 64;
    const unsigned grid = static_cast<unsigned>(std::min<int64_t>(65536, (items + 255) / 256));
    hipLaunchKernelGGL(pack_nvfp4_codes_kernel, dim3(grid), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(w), static_cast<int64_t>(E), N,
                       static_cast<int64_t>(K / 2), half, static_cast<uint8_t*>(out));
    hipLaunchKernelGGL(pack_nvfp4_scales_kernel, dim3(grid), dim3(256), 0, stream, w_scales,
                       static_cast<int64_t>(E), N, static_cast<int64_t>(K / 16), half, out_scales);
    return check_launch("moe_pack_weights");
  }
  const int bits = fmt == MOE_BF16 ? 16 : (fmt == MOE_MXFP8_E4M3 ? 8 : 4);
  const int64_t kbytes = static_cast<int64_t>(K) * bits / 8;
  MOE_REQUIRE(N % 64 == 0 && kbytes % kStageBytes == 0, MOE_ERR_INVALID_ARG,
              "moe_pack_weights: need N % 64 == 0 and K a multiple of one 128-byte stage "
              "(64 bf16, 128 E4M3 or 256 E2M1 values)");
  MOE_REQUIRE(half == 0 || (half > 0 && N == 2 * half && half % 32 == 0), MOE_ERR_INVALID_ARG,
              "moe_pack_weights: gate/up pairing needs N == 2 * half and half % 32 == 0");
  MOE_REQUIRE(w && out && (fmt == MOE_BF16 || (w_scales && out_scales)), MOE_ERR_INVALID_ARG,
              "moe_pack_weights: null pointer");
  MOE_REQUIRE(aligned16(w) && aligned16(out), MOE_ERR_ALIGNMENT,
              "moe_pack_weights: w and out must be 16-byte aligned");
  const int64_t pieces = static_cast<int64_t>(E) * N * kbytes / 16;
  const unsigned grid = static_cast<unsigned>(std::min<int64_t>(65536, (pieces + 255) / 256));
  hipLaunchKernelGGL(pack_codes_kernel, dim3(grid), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(w), static_cast<int64_t>(E), N, kbytes, half,
                     static_cast<uint8_t*>(out));
  if (fmt != MOE_BF16) {
    const int sub = fmt == MOE_MXFP8_E4M3 ? XOp<XOP_FP8>::kSub : XOp<XOP_FP4>::kSub;
    const int64_t nsc = static_cast<int64_t>(E) * N * (K / 32);
    const unsigned g2 = static_cast<unsigned>(std::min<int64_t>(65536, (nsc + 255) / 256));
    hipLaunchKernelGGL(pack_scales_kernel, dim3(g2), dim3(256), 0, stream, w_scales,
                       static_cast<int64_t>(E), N, static_cast<int64_t>(K / 32), sub, half,
                       out_scales);
  }
  return check_launch("moe_pack_weights");
}
