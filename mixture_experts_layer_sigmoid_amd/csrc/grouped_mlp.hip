// moe_grouped_mlp_fwd: grouped fc1 + SwiGLU (+ MX quantization of h), then
// grouped fc2, over expert-major row segments.
//
// Page "[PyTorch] DeepSeekV3Layer: full MoE transformer layer (MLA +
// DeepSeek MoE)": Description (experts as GroupedLinear -> ScaledSwiGLU ->
// GroupedLinear, fused into one grouped MLP) and Performance section ("Where
// the time goes": fused grouped MLP, fc1+SwiGLU fwd and fc2 fwd, MXFP8).
// Page "Mistral Large 3 NVFP4 TRTLLM MoE support", Highlights: fc1's weight
// holds the w1 (gate) and w3 (up) halves; here rows [0, F) gate, [F, 2F) up.
//
// Kernel design (gfx950):
//   * One persistent kernel per GEMM. A tile is (expert e, row block m,
//     column block n): up to MMAX rows of the expert's segment against 128
//     weight rows. Every workgroup builds the tile list from `offsets` in
//     LDS (m-tiles per expert, prefix sum), so no host round trip is needed.
//     Tiles are ordered expert-major, then column block, then row block, and
//     the list is cut into 8 contiguous chunks, one per XCD (workgroups are
//     dispatched to XCDs round-robin by index). The workgroups of one XCD
//     thus run consecutive tiles together: the column blocks of one expert
//     share its activation rows in that XCD's L2, and the row blocks of one
//     weight tile (experts with more than MMAX rows) run side by side, so
//     each weight byte comes from HBM once.
//   * Both operands stream into LDS with direct global->LDS 16-byte loads
//     (no register staging), STAGES deep. Each stage holds 128 bytes of K
//     per row: 64 bf16, 128 E4M3 or 256 E2M1 values. Rows are stored with
//     their eight 16-byte chunks XOR-swizzled by (row % 8), which keeps the
//     MFMA operand reads (8 rows x 16 bytes per lane group) free of bank
//     conflicts. MX block scales (one byte per 32 values) get their own
//     small LDS arrays.
//   * 4 wavefronts; wavefront w owns 32 weight rows (one 32x32 MFMA column
//     block) and every row block of the tile, so each weight element is read
//     from LDS once per row block and all four SIMDs stay busy whatever the
//     row count. MFMA: 32x32x16 bf16, or the block-scaled 32x32x64 f8f6f4
//     with E4M3 / E2M1 operands and E8M0 scales.
//   * fc1 tiles pair 64 gate columns with the matching 64 up columns: wave w
//     holds gate columns [16w, 16w+16) in its MFMA columns 0..15 and the
//     same up columns in 16..31, so SwiGLU needs one lane exchange. h goes
//     through LDS to coalesced bf16 stores or to the MX encoder (whole
//     32-column blocks per row).
//   * fc2 tiles store y (bf16) through LDS as full 16-byte row chunks.
#include "common.h"
#include "mx_codec.h"
#include "gemm_util.h"
#include "expert_gemm.h"

#include <algorithm>
#include <type_traits>

namespace moe {
namespace {

constexpr int kMaxGroups = 1024;

enum { OP_BF16 = 0, OP_FP8 = 1, OP_FP4 = 2 };
enum { EPI_SWIGLU = 0, EPI_PLAIN = 1, EPI_DSWIGLU = 2 };

// Per-format constants for RB bytes of K per row per stage: MFMA k-steps per
// stage (32x32x16 bf16 consumes 32 bytes of K per row, 32x32x64 E4M3 64
// bytes, 32x32x64 E2M1 32 bytes) and MX scale bytes per row per stage (one
// per 32 elements).
template <int OP, int RB>
struct Op {
  static constexpr int kSub = OP == OP_FP8 ? RB / 64 : RB / 32;
  static constexpr int kScaleBytes = OP == OP_BF16 ? 0 : (OP == OP_FP8 ? RB / 32 : RB / 16);
};

struct Args {
  const uint8_t* a;        // activation rows (or token rows with gather)
  int64_t a_row_bytes;
  const uint8_t* a_sc;     // MX scales of a
  int64_t a_sc_row_bytes;
  const int32_t* gather;   // optional row -> source row (-1: padding)
  const uint8_t* b;        // weights of expert 0
  int64_t b_exp_bytes;
  int64_t b_row_bytes;
  const uint8_t* b_sc;
  int64_t b_sc_exp_bytes;
  int64_t b_sc_row_bytes;
  int up_row;              // fc1: first row of the up half (F)
  const int32_t* offsets;  // [E+1]
  int E;
  int64_t rows;            // rows of a / out (bound)
  int n_blocks;            // column blocks per expert
  int k_stages;            // K bytes / 128
  uint8_t* out;
  int64_t out_row_bytes;
  uint8_t* out_sc;
  int64_t out_sc_row_bytes;
  float* act_save;         // optional [rows, 2F] fp32 (fc1 only)
  int act_cols;            // 2F
  // EPI_DSWIGLU
  const float* a_saved;    // saved fc1 output A [rows, 2F] fp32 (gate | up)
  float* da_f32;           // optional fp32 copy of dA [rows, 2F]
};

template <int MMAX, int STAGES, int NCB, int OP, int RB>
struct Smem {
  static constexpr int kBRows = 128 * NCB;
  static constexpr int kA = MMAX * RB;
  static constexpr int kB = kBRows * RB;
  static constexpr int kASc = MMAX * Op<OP, RB>::kScaleBytes;
  static constexpr int kBSc = kBRows * Op<OP, RB>::kScaleBytes;
  static constexpr int kStage = kA + kB + kASc + kBSc;
  static constexpr int kSched = (kMaxGroups + 2) * 4 + MMAX * 4;
  static constexpr int kTotal = STAGES * kStage + kSched;
};

// Weight row that tile row `br` streams. fc1 (SwiGLU): tile rows come in
// groups of 32 = 16 gate rows then the matching 16 up rows, group q covering
// h columns [16q, 16q+16) of the tile; fc2: consecutive output rows.
template <int EPI, int NCB>
__device__ __forceinline__ int weight_row(int nblk, int br, int up_row) {
  if (EPI == EPI_SWIGLU) {
    const int q = br >> 5, within = br & 31;
    return nblk * (64 * NCB) + 16 * q + (within & 15) + (within >= 16 ? up_row : 0);
  }
  return nblk * (128 * NCB) + br;
}

// MMAX:   rows per tile (multiple of 32 * WM, <= 256)
// STAGES: pipeline depth
// RB:     bytes of K per row per stage (128 or 64)
// NCB:    32-column MFMA blocks per wavefront (tile = 128 * NCB weight rows)
// WM:     wavefront groups along the rows (4 * WM wavefronts; wave w owns
//         column group w % 4 and row blocks w / 4, w / 4 + WM, ...)
// OCC:    workgroups resident per CU (persistent grid = 256 * OCC)
template <int MMAX, int STAGES, int NCB, int WM, int OCC, int RB, int OP, int EPI, int OUTF>
__global__ __launch_bounds__(256 * WM) __attribute__((amdgpu_waves_per_eu(OCC * WM, OCC * WM)))
void grouped_gemm_kernel(Args p) {
  using S = Smem<MMAX, STAGES, NCB, OP, RB>;
  using O = Op<OP, RB>;
  constexpr int kCpr = RB / 16;         // 16-byte chunks per row per stage
  constexpr int kRpi = 1024 / RB;       // rows per 1 KB direct-load instruction
  constexpr int NT = 256 * WM;          // threads
  constexpr int NW = 4 * WM;            // wavefronts
  constexpr int kRB = MMAX / 32;        // row blocks per tile
  constexpr int kRBW = kRB / WM;        // row blocks per wavefront
  static_assert(kRB % WM == 0, "row blocks must split evenly over the wave groups");
  constexpr int kSB = O::kScaleBytes;
  static_assert(kSB % 4 == 0, "MX scales are staged as whole dwords per row");
  constexpr int kBR = S::kBRows;        // weight rows per tile
  constexpr int kAIns = MMAX / (kRpi * NW);  // A load instructions per wave per stage
  constexpr int kBIns = kBR / (kRpi * NW);   // B load instructions per wave per stage
  static_assert(kAIns >= 1 && kBIns >= 1, "tile too small for the wavefront count");
  __shared__ __attribute__((aligned(16))) uint8_t smem[S::kTotal];
  int32_t* s_mt = reinterpret_cast<int32_t*>(smem + STAGES * S::kStage);   // [E+1] m-tile prefix
  int32_t* s_src = s_mt + (kMaxGroups + 1);                                  // [MMAX] source rows
  int32_t* s_tot = s_src + MMAX;
  // [NT] scan scratch; aliases the stage buffers, which the tile-list scan
  // finishes with before the first load is issued
  int32_t* part = reinterpret_cast<int32_t*>(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wn = wave & 3, wm = wave >> 2;
  const int E = p.E;

  // ---- tile list: m-tiles per expert, inclusive prefix in s_mt[1..E] ----
  {
    const int per = (E + NT - 1) / NT;
    const int lo = tid * per, hi = min(E, lo + per);
    int s = 0;
    for (int e = lo; e < hi; ++e) {
      int n_e = min(p.offsets[e + 1], (int)p.rows) - p.offsets[e];
      n_e = n_e < 0 ? 0 : n_e;
      const int mt = (n_e + MMAX - 1) / MMAX;
      s_mt[e + 1] = mt;
      s += mt;
    }
    part[tid] = s;
    __syncthreads();
    for (int d = 1; d < NT; d <<= 1) {
      const int v = tid >= d ? part[tid - d] : 0;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    int run = tid > 0 ? part[tid - 1] : 0;
    for (int e = lo; e < hi; ++e) {
      run += s_mt[e + 1];
      s_mt[e + 1] = run;
    }
    if (tid == 0) {
      s_mt[0] = 0;
      s_tot[0] = part[NT - 1];
    }
    __syncthreads();
  }
  // the tile list is cut into 8 contiguous chunks, one per XCD
  const int64_t total_tiles = static_cast<int64_t>(s_tot[0]) * p.n_blocks;
  const XcdSlot xs = xcd_slot();
  const int64_t t_first = total_tiles * xs.xcd / kNumXcd + xs.slot;
  const int64_t t_end = total_tiles * (xs.xcd + 1) / kNumXcd;

  for (int64_t t = t_first; t < t_end; t += xs.nslots) {
    int e, nblk, mblk, row0, nrows, KT;
    {
      // ---- decode: expert e (s_mt[e]*nb <= t < s_mt[e+1]*nb), then column
      // block (slow) and row block (fast) inside the expert ----
      int lo = 0, hi = E;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (static_cast<int64_t>(s_mt[mid]) * p.n_blocks <= t) lo = mid;
        else hi = mid;
      }
      e = lo;
      const int mtiles = s_mt[e + 1] - s_mt[e];
      const int64_t local = t - static_cast<int64_t>(s_mt[e]) * p.n_blocks;
      nblk = static_cast<int>(local / mtiles);
      mblk = static_cast<int>(local % mtiles);
      const int seg_lo = p.offsets[e];
      const int n_e = min(p.offsets[e + 1], (int)p.rows) - seg_lo;
      // full MMAX-row tiles first, the remainder last (MFMA padding only in
      // the last tile's final 32-row block)
      row0 = seg_lo + mblk * MMAX;
      nrows = min(MMAX, n_e - mblk * MMAX);
      KT = p.k_stages;
    }
    if (nrows <= 0) continue;  // uniform across the workgroup
    const int nrb = (nrows + 31) >> 5;

    // ---- per-lane global sources of this tile's loads ----
    const uint8_t* a_src[kAIns];
#pragma unroll
    for (int i = 0; i < kAIns; ++i) {
      const int r = kRpi * (wave + NW * i) + lane / kCpr;
      int src = row0 + min(r, nrows - 1);
      if (p.gather) {
        src = p.gather[src];
        if (src < 0) src = 0;  // padding row: loads any valid row, h is zeroed
      }
      a_src[i] = p.a + static_cast<int64_t>(src) * p.a_row_bytes +
                 (((lane % kCpr) ^ swz_key<RB>(r)) << 4);
    }
    if (p.gather && EPI == EPI_SWIGLU) {
      for (int r = tid; r < MMAX; r += NT) s_src[r] = r < nrows ? p.gather[row0 + r] : 0;
    }
    const uint8_t* b_src[kBIns];
    const uint8_t* bexp = p.b + static_cast<int64_t>(e) * p.b_exp_bytes;
#pragma unroll
    for (int i = 0; i < kBIns; ++i) {
      const int br = kRpi * (wave + NW * i) + lane / kCpr;
      const int wrow = weight_row<EPI, NCB>(nblk, br, p.up_row);
      b_src[i] = bexp + static_cast<int64_t>(wrow) * p.b_row_bytes + (((lane % kCpr) ^ swz_key<RB>(br)) << 4);
    }
    // ---- MX scale sources: kSB bytes (kSB/4 dwords) per row per stage; one
    // 4-byte direct load per lane, 64/(kSB/4) rows per instruction ----
    constexpr int kDpr = kSB > 0 ? kSB / 4 : 1;
    constexpr int kScRows = 64 / kDpr;                 // rows per scale instruction
    constexpr int kAScIns = kSB > 0 ? MMAX / kScRows : 1;
    constexpr int kBScIns = kSB > 0 ? kBR / kScRows : 1;
    const uint8_t* asc_src[(kAScIns + NW - 1) / NW];
    const uint8_t* bsc_src[(kBScIns + NW - 1) / NW];
    if (kSB > 0) {
#pragma unroll
      for (int q = 0; q < (kAScIns + NW - 1) / NW; ++q) {
        const int j = wave + NW * q;
        const int r = min(j * kScRows + lane / kDpr, nrows - 1);
        int src = row0 + r;
        if (p.gather) {
          src = p.gather[src];
          if (src < 0) src = 0;
        }
        asc_src[q] = p.a_sc + static_cast<int64_t>(src) * p.a_sc_row_bytes + (lane % kDpr) * 4;
      }
      const uint8_t* bsexp = p.b_sc + static_cast<int64_t>(e) * p.b_sc_exp_bytes;
#pragma unroll
      for (int q = 0; q < (kBScIns + NW - 1) / NW; ++q) {
        const int r = min((wave + NW * q) * kScRows + lane / kDpr, kBR - 1);
        const int wrow = weight_row<EPI, NCB>(nblk, r, p.up_row);
        bsc_src[q] = bsexp + static_cast<int64_t>(wrow) * p.b_sc_row_bytes + (lane % kDpr) * 4;
      }
    }

    f32x16_t acc[kRBW][NCB];
#pragma unroll
    for (int i = 0; i < kRBW; ++i)
#pragma unroll
      for (int c = 0; c < NCB; ++c) acc[i][c] = f32x16_t{};

    // vector-memory instructions this wave issues per stage: A instruction i
    // covers rows [8*(wave+4i), +8) and is issued when that range starts
    // below nrows; scale instruction j covers rows [j*kScRows, ...)
    int my_a = 0;
#pragma unroll
    for (int i = 0; i < kAIns; ++i) my_a += (kRpi * (wave + NW * i) < nrows) ? 1 : 0;
    int my_asc = 0, my_bsc = 0;
    if (kSB > 0) {
#pragma unroll
      for (int q = 0; q < (kAScIns + NW - 1) / NW; ++q)
        my_asc += ((wave + NW * q) < kAScIns && (wave + NW * q) * kScRows < nrows) ? 1 : 0;
#pragma unroll
      for (int q = 0; q < (kBScIns + NW - 1) / NW; ++q) my_bsc += ((wave + NW * q) < kBScIns) ? 1 : 0;
    }
    const int per_stage = my_a + kBIns + my_asc + my_bsc;

    auto issue = [&](int kt) {
      uint8_t* st = smem + (kt % STAGES) * S::kStage;
      const int64_t kb = static_cast<int64_t>(kt) * RB;
#pragma unroll
      for (int i = 0; i < kBIns; ++i) lds_load16(b_src[i] + kb, st + S::kA + (wave + NW * i) * 1024);
#pragma unroll
      for (int i = 0; i < kAIns; ++i)
        if (kRpi * (wave + NW * i) < nrows) lds_load16(a_src[i] + kb, st + (wave + NW * i) * 1024);
      if (kSB > 0) {
        const int64_t ks = static_cast<int64_t>(kt) * kSB;
#pragma unroll
        for (int q = 0; q < (kAScIns + NW - 1) / NW; ++q) {
          const int j = wave + NW * q;
          if (j < kAScIns && j * kScRows < nrows) lds_load4(asc_src[q] + ks, st + S::kA + S::kB + j * 256);
        }
#pragma unroll
        for (int q = 0; q < (kBScIns + NW - 1) / NW; ++q) {
          const int j = wave + NW * q;
          if (j < kBScIns) lds_load4(bsc_src[q] + ks, st + S::kA + S::kB + S::kASc + j * 256);
        }
      }
    };

#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < KT) issue(s);

    // number of this wave's row blocks (mb = wm, wm + WM, ...) that hold rows
    const int nv = nrb > wm ? min(kRBW, (nrb - wm + WM - 1) / WM) : 0;
    const int g = lane >> 5;

    // One stage of MFMAs for the first NV row blocks of this wave. Operands of
    // k-step s+1 are read from LDS before the MFMAs of k-step s are issued,
    // so LDS latency overlaps the matrix cores.
    auto stage_mfma = [&](const uint8_t* st, auto nv_c) {
      constexpr int NV = decltype(nv_c)::value;
      const uint8_t* sa = st;
      const uint8_t* sb = st + S::kA;
      if constexpr (OP == OP_BF16) {
        bf16x8_t ao[2][NV > 0 ? NV : 1], bo[2][NCB];
        auto load = [&](int s, int buf) {
#pragma unroll
          for (int c = 0; c < NCB; ++c)
            bo[buf][c] = *reinterpret_cast<const bf16x8_t*>(sb + swz<RB>(32 * (wn * NCB + c) + (lane & 31), 2 * s + g));
#pragma unroll
          for (int i = 0; i < NV; ++i)
            ao[buf][i] = *reinterpret_cast<const bf16x8_t*>(sa + swz<RB>((wm + WM * i) * 32 + (lane & 31), 2 * s + g));
        };
        load(0, 0);
#pragma unroll
        for (int s = 0; s < O::kSub; ++s) {
          if (s + 1 < O::kSub) load(s + 1, (s + 1) & 1);
#pragma unroll
          for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int c = 0; c < NCB; ++c)
              acc[i][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao[s & 1][i], bo[s & 1][c], acc[i][c], 0, 0, 0);
        }
      } else {
        constexpr int dpr = kSB > 0 ? kSB / 4 : 1;
        const uint32_t* sasc = reinterpret_cast<const uint32_t*>(st + S::kA + S::kB);
        const uint32_t* sbsc = reinterpret_cast<const uint32_t*>(st + S::kA + S::kB + S::kASc);
        uint32_t bsc[NCB][dpr], asc[NV > 0 ? NV : 1][dpr];
#pragma unroll
        for (int c = 0; c < NCB; ++c)
#pragma unroll
          for (int d = 0; d < dpr; ++d) bsc[c][d] = sbsc[(32 * (wn * NCB + c) + (lane & 31)) * dpr + d];
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
          for (int d = 0; d < dpr; ++d) asc[i][d] = sasc[((wm + WM * i) * 32 + (lane & 31)) * dpr + d];
        i32x8_t ao[2][NV > 0 ? NV : 1], bo[2][NCB];
        auto opnd = [&](const uint8_t* base, int row, int s) -> i32x8_t {
          if (OP == OP_FP8) {
            const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(base + swz<RB>(row, 4 * s + g));
            const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(base + swz<RB>(row, 4 * s + 2 + g));
            return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                           (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          }
          // E2M1, 32x32x64: lane group g holds k [32g, 32g+32) (16 bytes)
          const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(base + swz<RB>(row, 2 * s + g));
          return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], 0, 0, 0, 0};
        };
        auto load = [&](int s, int buf) {
#pragma unroll
          for (int c = 0; c < NCB; ++c) bo[buf][c] = opnd(sb, 32 * (wn * NCB + c) + (lane & 31), s);
#pragma unroll
          for (int i = 0; i < NV; ++i) ao[buf][i] = opnd(sa, (wm + WM * i) * 32 + (lane & 31), s);
        };
        constexpr int kSub = O::kSub;
        load(0, 0);
#pragma unroll
        for (int s = 0; s < kSub; ++s) {
          if (s + 1 < kSub) load(s + 1, (s + 1) & 1);
          // k-step s covers MX blocks 2s and 2s+1 of the stage; lane group g
          // supplies the scale of block 2s+g in the low byte of its operand
          const int blk = 2 * s + g;
          const int bw = blk >> 2, bsh = 8 * (blk & 3);
#pragma unroll
          for (int i = 0; i < NV; ++i) {
            const int as = static_cast<int>((asc[i][bw] >> bsh) & 0xFFu);
#pragma unroll
            for (int c = 0; c < NCB; ++c) {
              const int bs = static_cast<int>((bsc[c][bw] >> bsh) & 0xFFu);
              if (OP == OP_FP8)
                acc[i][c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ao[s & 1][i], bo[s & 1][c], acc[i][c], 0, 0, 0, as, 0, bs);
              else
                acc[i][c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ao[s & 1][i], bo[s & 1][c], acc[i][c], 4, 4, 0, as, 0, bs);
            }
          }
        }
      }
    };

    for (int kt = 0; kt < KT; ++kt) {
      // stages issued after kt that may stay in flight
      const int ahead = min(STAGES - 2, KT - 1 - kt);
      wait_vm(ahead * per_stage);
      // every wave's loads of stage kt have landed; LDS reads of stage kt-1
      // are done (the load below reuses that buffer)
      lds_barrier();
      if (kt + STAGES - 1 < KT) issue(kt + STAGES - 1);
      const uint8_t* st = smem + (kt % STAGES) * S::kStage;
      switch (nv) {
#define MOE_NV(N) case N: if constexpr (N <= kRBW) stage_mfma(st, std::integral_constant<int, N>{}); break;
        MOE_NV(1) MOE_NV(2) MOE_NV(3) MOE_NV(4) MOE_NV(5) MOE_NV(6) MOE_NV(7) MOE_NV(8)
#undef MOE_NV
        default: break;
      }
    }
    __syncthreads();  // all waves done with the stage buffers

    // ---- epilogue: accumulators -> LDS tile [rows][kCs] fp32, then a
    // row-major pass (SwiGLU / act save / MX encode / bf16) with 16-byte
    // global stores ----
    // C layout of a 32x32 MFMA: lane l, element r -> row 8*(r/4) + 4*(l/32) + r%4, column l%32
    constexpr int kCs = kBR + 4;  // padded row stride (floats)
    static_assert(MMAX * kCs * 4 <= STAGES * S::kStage, "epilogue tile must fit the stage buffers");
    float* cs = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int i = 0; i < kRBW; ++i) {
      const int mb = wm + WM * i;
      if (mb < nrb) {
#pragma unroll
        for (int c = 0; c < NCB; ++c) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            cs[row * kCs + 32 * (wn * NCB + c) + (lane & 31)] = acc[i][c][r];
          }
        }
      }
    }
    __syncthreads();
    if constexpr (EPI == EPI_SWIGLU) {
      // h column c (0..64*NCB) of this tile: gate at tile column
      // 32*(c/16) + c%16, up at the same + 16
      constexpr int kHc = 64 * NCB;
      if constexpr (OUTF == MOE_BF16) {
        for (int i = tid; i < nrows * (kHc / 8); i += NT) {
          const int row = i / (kHc / 8), c0 = (i % (kHc / 8)) * 8;
          const bool zero = p.gather && s_src[row] < 0;
          const float* gp = cs + row * kCs + 32 * (c0 >> 4) + (c0 & 15);
          const float* up = gp + 16;
          float h[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) h[q] = zero ? 0.f : silu_mul(gp[q], up[q]);
          const int64_t grow = row0 + row;
          *reinterpret_cast<u32x4_t*>(p.out + grow * p.out_row_bytes + (nblk * kHc + c0) * 2) =
              u32x4_t{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]), pack_bf16x2(h[4], h[5]),
                      pack_bf16x2(h[6], h[7])};
          if (p.act_save) {
            float* ar = p.act_save + grow * p.act_cols + nblk * kHc + c0;
            store8_f32(ar, gp);
            store8_f32(ar + p.up_row, up);
          }
        }
      } else {
        constexpr bool fp4 = OUTF == MOE_MXFP4_E2M1;
        constexpr int kBlk = kHc / 32;  // 32-column MX blocks per row of the tile
        for (int i = tid; i < nrows * kBlk; i += NT) {
          const int row = i / kBlk, blk = i % kBlk;
          const bool zero = p.gather && s_src[row] < 0;
          float v[32];
#pragma unroll
          for (int q = 0; q < 32; ++q) {
            const int c = blk * 32 + q;
            const float* gp = cs + row * kCs + 32 * (c >> 4) + (c & 15);
            v[q] = zero ? 0.f : silu_mul(gp[0], gp[16]);
          }
          uint32_t words[8];
          const uint32_t sb = mx_encode_block<fp4>(v, words);
          const int64_t r = row0 + row;
          const int gblk = nblk * kBlk + blk;
          if (fp4) {
            *reinterpret_cast<u32x4_t*>(p.out + r * p.out_row_bytes + gblk * 16) =
                u32x4_t{words[0], words[1], words[2], words[3]};
          } else {
            u32x4_t* o = reinterpret_cast<u32x4_t*>(p.out + r * p.out_row_bytes + gblk * 32);
            o[0] = u32x4_t{words[0], words[1], words[2], words[3]};
            o[1] = u32x4_t{words[4], words[5], words[6], words[7]};
          }
          p.out_sc[r * p.out_sc_row_bytes + gblk] = static_cast<uint8_t>(sb);
          if (p.act_save) {
            for (int q = 0; q < 32; q += 8) {
              const int c = blk * 32 + q;
              const float* gp = cs + row * kCs + 32 * (c >> 4) + (c & 15);
              float* ar = p.act_save + r * p.act_cols + nblk * kHc + c;
              store8_f32(ar, gp);
              store8_f32(ar + p.up_row, gp + 16);
            }
          }
        }
      }
    } else if constexpr (EPI == EPI_PLAIN) {
      uint8_t* obase = p.out;
      for (int i = tid; i < nrows * (kBR / 8); i += NT) {
        const int row = i / (kBR / 8), c0 = (i % (kBR / 8)) * 8;
        const float* v = cs + row * kCs + c0;
        *reinterpret_cast<u32x4_t*>(obase + static_cast<int64_t>(row0 + row) * p.out_row_bytes +
                                    (static_cast<int64_t>(nblk) * kBR + c0) * 2) =
            u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                    pack_bf16x2(v[6], v[7])};
      }
    } else {
      // dSwiGLU: the tile holds dH for columns [nblk*kBR, +kBR) of F; with the
      // saved fc1 output (g | u) it gives dA = [dgate | dup]:
      //   dgate = dH * u * sig(g) * (1 + g * (1 - sig(g))),  dup = dH * silu(g)
      const int F = p.up_row;
      const int64_t a2 = 2ll * F;  // elements per saved / dA row
      if constexpr (OUTF == MOE_BF16) {
        for (int i = tid; i < nrows * (kBR / 8); i += NT) {
          const int row = i / (kBR / 8), c0 = (i % (kBR / 8)) * 8;
          const int col = nblk * kBR + c0;
          const int64_t grow = row0 + row;
          float gv[8], uv[8], dg[8], du[8];
          load8_f32(p.a_saved + grow * a2 + col, gv);
          load8_f32(p.a_saved + grow * a2 + F + col, uv);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float g = gv[q], u = uv[q];
            const float dh = cs[row * kCs + c0 + q];
            const float sig = 1.f / (1.f + expf(-g));
            dg[q] = dh * u * sig * (1.f + g * (1.f - sig));
            du[q] = dh * (g * sig);
          }
          uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + grow * a2;
          *reinterpret_cast<u32x4_t*>(o + col) =
              u32x4_t{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]), pack_bf16x2(dg[4], dg[5]),
                      pack_bf16x2(dg[6], dg[7])};
          *reinterpret_cast<u32x4_t*>(o + F + col) =
              u32x4_t{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]), pack_bf16x2(du[4], du[5]),
                      pack_bf16x2(du[6], du[7])};
        }
      } else {
        constexpr bool fp4 = OUTF == MOE_MXFP4_E2M1;
        constexpr int kBlkBytes = fp4 ? 16 : 32;
        for (int i = tid; i < nrows * (kBR / 32); i += NT) {
          const int row = i / (kBR / 32), blk = i % (kBR / 32);
          const int col = nblk * kBR + blk * 32;
          const int64_t grow = row0 + row;
          float dg[32], du[32];
#pragma unroll
          for (int w8 = 0; w8 < 4; ++w8) {
            float gv[8], uv[8];
            load8_f32(p.a_saved + grow * a2 + col + w8 * 8, gv);
            load8_f32(p.a_saved + grow * a2 + F + col + w8 * 8, uv);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const float g = gv[q], u = uv[q];
              const float dh = cs[row * kCs + blk * 32 + w8 * 8 + q];
              const float sig = 1.f / (1.f + expf(-g));
              dg[w8 * 8 + q] = dh * u * sig * (1.f + g * (1.f - sig));
              du[w8 * 8 + q] = dh * (g * sig);
            }
          }
          uint32_t words[8];
          uint8_t* orow = p.out + grow * p.out_row_bytes;
          uint8_t* srow = p.out_sc + grow * p.out_sc_row_bytes;
#pragma unroll
          for (int part = 0; part < 2; ++part) {
            const float* v = part ? du : dg;
            const int c = part ? F + col : col;
            const uint32_t sb = mx_encode_block<fp4>(v, words);
            u32x4_t* o = reinterpret_cast<u32x4_t*>(orow + (c / 32) * kBlkBytes);
            o[0] = u32x4_t{words[0], words[1], words[2], words[3]};
            if (!fp4) o[1] = u32x4_t{words[4], words[5], words[6], words[7]};
            srow[c / 32] = static_cast<uint8_t>(sb);
            if (p.da_f32) {
              float* ob = p.da_f32 + grow * a2 + c;
#pragma unroll
              for (int w8 = 0; w8 < 4; ++w8) store8_f32(ob + w8 * 8, v + w8 * 8);
            }
          }
        }
      }
    }
    __syncthreads();  // LDS reused by the next tile
  }
}

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

template <int MMAX, int STAGES, int NCB, int WM, int OCC, int RB, int OP, int EPI, int OUTF>
int launch_gemm(Args a, hipStream_t stream) {
  a.n_blocks /= NCB;
  a.k_stages = static_cast<int>(a.a_row_bytes / RB);
  const int grid = kNumCu * OCC;  // persistent: OCC workgroups per CU
  hipLaunchKernelGGL((grouped_gemm_kernel<MMAX, STAGES, NCB, WM, OCC, RB, OP, EPI, OUTF>), dim3(grid),
                     dim3(256 * WM), 0, stream, a);
  return check_launch("grouped GEMM");
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
