// moe_grouped_wgrad: per-expert weight gradients dW[e] = A_e^T B_e over
// the expert's K segment (its token rows), MXFP8 operands, bf16 output.
//
// Page "[PyTorch] DeepSeekV3Layer: full MoE transformer layer (MLA +
// DeepSeek MoE)", Performance section, "Where the time goes": the wgrad of
// the fused grouped MLP in MXFP8.
//
// Shape of the work: one output matrix of M x N bf16 per expert (for a
// 384-expert layer about 50 GB of dW per step) against K segments that are
// mostly one or two 128-element blocks long and, under a skewed router, a few
// thousand long for a handful of experts. The kernel is therefore built
// around a continuous stream of output stores, not around the contraction:
//   * Persistent grid, OCC workgroups of 4 wavefronts per CU. A tile is
//     (expert, 128 dW rows, 128 dW columns); its K segment is consumed in
//     stages of 128 E4M3 values per row (16 KB per operand + scales).
//   * Every workgroup walks a flat sequence of (tile, stage) items through a
//     two-buffer LDS ring: the loads of item i+1 are issued before item i is
//     computed, and a finished tile's output is staged (bf16) in the buffer
//     that tile just consumed, then written with 16-byte row stores. The
//     stores are never waited for explicitly: the next wait is for loads
//     issued before them, so they drain while the following item runs.
//   * Schedule over the 8 XCDs (workgroups are dispatched to XCDs
//     round-robin by index): experts whose segment has at most 8 stages go
//     whole to one XCD (the experts are cut into 8 contiguous runs of about
//     equal cost), so an XCD reads their operands once; the dW rows of each
//     longer expert are split into 8 slices, one per XCD, and run first, so
//     the skewed K lengths stay balanced across the chip. Inside an XCD the
//     tiles run expert by expert in groups of 8 row blocks; concurrent tiles
//     share their operand blocks in that XCD's L2.
//   * Operands come in the stage-major layout the segment quantizer writes
//     ([stage][channel][128 K bytes], scales [stage][channel][4]): the
//     128-channel block of one stage that a tile loads is 16 KB of
//     contiguous memory, so its lines map evenly onto the L2 and HBM.
//   * MFMA 32x32x64 E4M3 with E8M0 block scales. The product is formed as
//     dW^T (bt rows as the MFMA's A operand), so each lane's accumulator
//     registers hold 4 consecutive dW columns of one dW row: the bf16 pack
//     is lane-local and the LDS staging writes are 8 bytes wide.
#include "common.h"
#include "gemm_util.h"

namespace moe {
namespace {

constexpr int kTile = 128;     // dW rows and columns per tile
constexpr int kRB = 128;       // K bytes (E4M3 values) per operand row per stage
constexpr int kMaxE = 1024;
constexpr int kOcc = 2;        // workgroups per CU
constexpr int kNT = 256;       // threads per workgroup

// LDS operand slots: two for A blocks, two for B blocks; a slot holds one
// 128-row block of one stage, codes [128][128] then scales [128][4].
constexpr int kCodes = kTile * kRB;            // 16 KB
constexpr int kSlot = kCodes + kTile * 4;
// schedule tables after the two buffers: segment starts [E+1] int32, then
// the split experts and this XCD's whole experts as int16 lists
constexpr int kSchedOfs = 4 * kSlot;
constexpr int kSmem = kSchedOfs + (kMaxE + 1) * 4 + 2 * kMaxE * 2;
// An expert whose segment has more than kWideKT stages is split across all
// XCDs by dW row blocks; shorter ones go whole to one XCD. Scheduling cost
// of a tile: kStoreCost for its 32 KB of output plus one per stage.
constexpr int kWideKT = 8;
constexpr int kStoreCost = 4;
constexpr int kGroup = 8;  // row blocks per group of the tile order
static_assert(kOcc * kSmem <= 160 * 1024, "LDS budget of a CU");

// 16-byte LDS store written as an instruction of its own: the compiler
// orders a plain LDS store after every direct global->LDS load in flight (it
// cannot tell the buffers apart) and would wait for the next stage's loads
// and the previous tile's stores. The target lies in the buffer the tile's
// last stage was read from, which no load in flight writes; the LDS reads
// that follow come from the same wave, which LDS executes in order.
__device__ __forceinline__ void ds_write16(uint8_t* lds, uint32_t a, uint32_t b, uint32_t c,
                                           uint32_t d) {
  const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const u32x4_t v = u32x4_t{a, b, c, d};
  asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

struct WArgs {
  const uint8_t* at;       // [KS][M][128] E4M3 (stage-major, see the entry point)
  const uint8_t* at_sc;    // [KS][M][4]
  const uint8_t* bt;       // [KS][N][128]
  const uint8_t* bt_sc;    // [KS][N][4]
  const int32_t* kofs;     // [E + 1] segment starts (multiples of 128)
  int E, M, N;
  uint8_t* dw;             // [E, M, N] bf16
  uint32_t at_bytes, at_sc_bytes, bt_bytes, bt_sc_bytes;  // operand sizes (< 4 GiB)
};

struct Tile {
  int e, m0, n0;   // expert, origin (dW rows m0.., columns n0..)
  int kt;          // stages of the expert's segment (0: empty, zeros)
  int g;           // global index of its first stage
};

__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(kOcc, kOcc)))
void wgrad_kernel(WArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmem];
  int32_t* s_kofs = reinterpret_cast<int32_t*>(smem + kSchedOfs);
  int16_t* s_wide = reinterpret_cast<int16_t*>(s_kofs + kMaxE + 1);
  int16_t* s_whole = s_wide + kMaxE;
  int32_t* s_scan = reinterpret_cast<int32_t*>(smem);  // [kNT + 1], before any load
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;   // wave's 64 x 64 quarter of the tile
  const int g = lane >> 5, l32 = lane & 31;

  for (int i = tid; i <= p.E; i += kNT) s_kofs[i] = p.kofs[i];
  __syncthreads();

  // ---- schedule (every workgroup derives its XCD's share) ----
  // Experts with at most kWideKT stages are whole units: they are cut into
  // 8 contiguous runs of about equal cost (in expert order), run x going to
  // XCD x, so each XCD reads the operands of its experts once and keeps them
  // in its L2 while it writes their dW. Longer experts are split: every XCD
  // takes its eighth of their dW row blocks and runs those tiles first.
  const XcdSlot xs = xcd_slot();
  const int E = p.E;
  const int mb = p.M / kTile, nb = p.N / kTile;
  const int per = (E + kNT - 1) / kNT;
  const int lo = min(E, tid * per), hi = min(E, lo + per);
  auto kt_of = [&](int e) { return (s_kofs[e + 1] - s_kofs[e]) / kRB; };
  // exclusive block scan of one int per thread; returns (prefix, total)
  auto scan = [&](int v, int& total) {
    s_scan[tid] = v;
    __syncthreads();
    for (int d = 1; d < kNT; d <<= 1) {
      const int t = tid >= d ? s_scan[tid - d] : 0;
      __syncthreads();
      s_scan[tid] += t;
      __syncthreads();
    }
    const int incl = s_scan[tid];
    total = s_scan[kNT - 1];
    __syncthreads();
    return incl - v;
  };
  int my_cost = 0, my_wide = 0;
  for (int e = lo; e < hi; ++e) {
    const int kt = kt_of(e);
    if (kt > kWideKT) ++my_wide;
    else my_cost += kStoreCost + max(kt, 1);
  }
  int total_cost, n_wide;
  int cost_pre = scan(my_cost, total_cost);
  int wide_pre = scan(my_wide, n_wide);
  // whole expert e goes to the XCD holding the middle of its cost interval
  auto xcd_of = [&](int pre, int c) {
    return min(kNumXcd - 1, static_cast<int>((2ll * pre + c) * kNumXcd / (2ll * max(total_cost, 1))));
  };
  int my_mine = 0;
  {
    int run = cost_pre;
    for (int e = lo; e < hi; ++e) {
      const int kt = kt_of(e);
      if (kt > kWideKT) continue;
      const int c = kStoreCost + max(kt, 1);
      if (xcd_of(run, c) == xs.xcd) ++my_mine;
      run += c;
    }
  }
  int n_whole;
  int mine_pre = scan(my_mine, n_whole);
  {
    int run = cost_pre;
    for (int e = lo; e < hi; ++e) {
      const int kt = kt_of(e);
      if (kt > kWideKT) {
        s_wide[wide_pre++] = static_cast<int16_t>(e);
        continue;
      }
      const int c = kStoreCost + max(kt, 1);
      if (xcd_of(run, c) == xs.xcd) s_whole[mine_pre++] = static_cast<int16_t>(e);
      run += c;
    }
  }
  __syncthreads();

  // tile list of this XCD: the split experts' tiles (rows [mlo, mhi) of
  // each), then its whole experts'. Inside an expert the tiles run in groups
  // of kGroup row blocks, each group column block by column block with the
  // row block fastest: the 64 tiles an XCD runs at once cover 8 row blocks x
  // 8 column blocks, and a group's 8 A blocks stay in L2 across the rounds
  // that sweep its columns (the output stream evicts anything older).
  // Workgroup slot s takes tiles s, s + nslots, ...; the position is kept
  // as (unit u, linear index rb * nb + cb) and stepped without division.
  const int mlo = mb * xs.xcd / kNumXcd, mhi = mb * (xs.xcd + 1) / kNumXcd;
  const int n_units = n_wide + n_whole;
  auto unit_rows = [&](int uu) { return uu < n_wide ? mhi - mlo : mb; };
  int u = 0, rb = xs.slot / nb, cb = xs.slot - (xs.slot / nb) * nb;
  const int drb = xs.nslots / nb, dcb = xs.nslots - drb * nb;
  auto settle = [&]() {  // carry rb into u; false past the last unit
    while (u < n_units && rb >= unit_rows(u)) {
      rb -= unit_rows(u);
      ++u;
    }
    return u < n_units;
  };
  auto current = [&]() {
    Tile t;
    t.e = u < n_wide ? s_wide[u] : s_whole[u - n_wide];
    // position r (column block fastest) in grouped order: groups of 8 row
    // blocks, inside a group the row block runs fastest
    const int r = rb * nb + cb;
    const int grp = r / (kGroup * nb);
    const int gm = min(kGroup, unit_rows(u) - kGroup * grp);
    const int idx = r - grp * kGroup * nb;
    const int cq = idx / gm;
    t.m0 = ((u < n_wide ? mlo : 0) + kGroup * grp + (idx - cq * gm)) * kTile;
    t.n0 = cq * kTile;
    const int k0 = s_kofs[t.e];
    t.kt = (s_kofs[t.e + 1] - k0) / kRB;
    t.g = k0 / kRB;
    return t;
  };
  auto step = [&]() {
    cb += dcb;
    rb += drb;
    if (cb >= nb) {
      cb -= nb;
      ++rb;
    }
    return settle();
  };
  if (!settle()) return;  // uniform: no tile for this workgroup

  // ---- per-lane load geometry (fixed across items) ----
  // codes: instruction q (0..15) of an operand covers tile rows [8q, 8q+8),
  // lane -> row 8q + lane/8, LDS slot lane%8 holding the row's logical chunk
  // (lane%8) ^ key(row); wave w issues q = w, w+4, w+8, w+12 of A and of B.
  int32_t ld_row[4], ld_chunk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * (wave + 4 * i) + (lane >> 3);
    ld_row[i] = r;
    ld_chunk[i] = ((lane & 7) ^ swz_key<kRB>(r)) << 4;
  }
  // scales: waves 0-1 load the A block's, waves 2-3 the B block's, 64 rows
  // x 4 bytes each
  const int sc_row = 64 * (wave & 1) + lane;

  // one operand block (128 channel rows of stage g) into a slot: 16 KB
  // contiguous in the stage-major layout; 4 loads per wave (+1 scale load)
  // (buffer-form direct-to-LDS loads: the LDS operand reads after them keep
  // exact waits, see gemm_util.h)
  const __amdgpu_buffer_rsrc_t at_rs = buf_rsrc(p.at, p.at_bytes), at_sc_rs = buf_rsrc(p.at_sc, p.at_sc_bytes);
  const __amdgpu_buffer_rsrc_t bt_rs = buf_rsrc(p.bt, p.bt_bytes), bt_sc_rs = buf_rsrc(p.bt_sc, p.bt_sc_bytes);
  auto issue_block = [&](__amdgpu_buffer_rsrc_t codes, __amdgpu_buffer_rsrc_t scl, uint32_t row0,
                         bool scl_wave, uint8_t* slot) {
    const uint32_t c = row0 * kRB;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      lds_load16_buf(codes, static_cast<uint32_t>(ld_row[i] * kRB + ld_chunk[i]), c,
                     slot + (wave + 4 * i) * 1024);
    if (scl_wave) lds_load4_buf(scl, static_cast<uint32_t>(sc_row * 4), row0 * 4, slot + kCodes + (wave & 1) * 256);
  };
  auto issue_a = [&](const Tile& t, int ks, uint8_t* slot) {
    issue_block(at_rs, at_sc_rs, static_cast<uint32_t>(t.g + ks) * p.M + t.m0, wave < 2, slot);
  };
  auto issue_b = [&](const Tile& t, int ks, uint8_t* slot) {
    issue_block(bt_rs, bt_sc_rs, static_cast<uint32_t>(t.g + ks) * p.N + t.n0, wave >= 2, slot);
  };

  f32x16_t acc[2][2];  // [dW row block mi][dW column block ni]
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x16_t{};

  // One stage: 2 k-steps of 64. MFMA A operand = bt rows (dW columns, the
  // accumulator's register index), B operand = at rows (dW rows, lanes).
  auto compute = [&](const uint8_t* sa, const uint8_t* sb) {
    const uint32_t* ssa = reinterpret_cast<const uint32_t*>(sa + kCodes);
    const uint32_t* ssb = reinterpret_cast<const uint32_t*>(sb + kCodes);
    uint32_t sca[2], scb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      sca[i] = ssa[64 * wm + 32 * i + l32];
      scb[i] = ssb[64 * wn + 32 * i + l32];
    }
    auto opnd = [&](const uint8_t* base, int row, int s) -> i32x8_t {
      const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(base + swz<kRB>(row, 4 * s + g));
      const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(base + swz<kRB>(row, 4 * s + 2 + g));
      return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    i32x8_t oa[2][2], ob[2][2];  // [k-step][block]
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        oa[s][i] = opnd(sa, 64 * wm + 32 * i + l32, s);
        ob[s][i] = opnd(sb, 64 * wn + 32 * i + l32, s);
      }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      // k-step s covers MX blocks 2s, 2s+1; lane group g supplies block 2s+g
      const int sh = 8 * (2 * s + g);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int as = static_cast<int>((sca[mi] >> sh) & 0xFFu);
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int bs = static_cast<int>((scb[ni] >> sh) & 0xFFu);
          acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              ob[s][ni], oa[s][mi], acc[mi][ni], 0, 0, 0, bs, 0, as);
        }
      }
    }
  };

  // Tile output, per wave (its 64 x 64 quarter), through its own 4 KB of the
  // B slot the tile's last stage was read from, in two rounds of 32 rows.
  // In a 32x32 block, lane l holds dW row l % 32 and, in registers
  // 4q..4q+3, dW columns 8q + 4g + 0..3 (g = l / 32); one permlane32 swap per
  // dword pair gives lane l < 32 columns [16p, 16p + 8) and lane l + 32
  // columns [16p + 8, 16p + 16) of the same row, written as 16 bytes into a
  // [32 rows][128 B] tile (16-byte chunks XOR-permuted by row % 8). Read back
  // as whole rows, each store covers 8 rows x 128 contiguous bytes of dW.
  auto epilogue = [&](const Tile& t, uint8_t* slot) {
    uint8_t* stg = slot + wave * 4096;
    uint8_t* out = p.dw + (static_cast<int64_t>(t.e) * p.M + t.m0 + 64 * wm) * p.N * 2 +
                   (t.n0 + 64 * wn) * 2;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const f32x16_t& a = acc[mi][ni];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const int q0 = 2 * pp, q1 = 2 * pp + 1;  // X: columns 8q0 + 4g.., Y: 8q1 + 4g..
          const uint32_t x0 = pack_bf16x2(a[4 * q0], a[4 * q0 + 1]);
          const uint32_t x1 = pack_bf16x2(a[4 * q0 + 2], a[4 * q0 + 3]);
          const uint32_t y0 = pack_bf16x2(a[4 * q1], a[4 * q1 + 1]);
          const uint32_t y1 = pack_bf16x2(a[4 * q1 + 2], a[4 * q1 + 3]);
          const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
          const int chunk = 4 * ni + 2 * pp + g;  // 16-byte chunk of the 128-byte row
          ds_write16(stg + l32 * 128 + ((chunk ^ (l32 & 7)) << 4), s0[0], s1[0], s0[1], s1[1]);
        }
      }
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int row = 8 * it + (lane >> 3), chunk = lane & 7;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stg + row * 128 + ((chunk ^ (row & 7)) << 4));
        __builtin_nontemporal_store(
            v, reinterpret_cast<u32x4_t*>(out + static_cast<int64_t>(32 * mi + row) * p.N * 2 + chunk * 16));
      }
    }
  };

  // ---- the item pipeline: (tile, stage) items, B blocks through two slots,
  // A blocks through two more, an A block that the next item shares (the
  // next tile of a group runs on the same dW rows) staying where it is ----
  // Per wave, in issue order: loads of item i+1, then the stores of the tile
  // item i ends; waiting for item i+1's loads leaves those stores in flight.
  Tile tc = current();
  bool tn_ok = step();
  Tile tn = tc;
  if (tn_ok) tn = current();
  int ks = 0, sa = 0, sb = 0;           // slots of the item being computed
  int a_e = -1, a_m0 = -1, a_g = -1;    // the A block loaded last (slot sa_last)
  int sa_last = 0;
  // loads of item (t, k) into B slot sb_next and, unless the last A block
  // loaded is the same one, the other A slot; returns its A slot
  auto issue = [&](const Tile& t, int k, int sb_next) {
    if (t.e != a_e || t.m0 != a_m0 || t.g + k != a_g) {
      sa_last ^= 1;
      issue_a(t, k, smem + sa_last * kSlot);
      a_e = t.e;
      a_m0 = t.m0;
      a_g = t.g + k;
    }
    issue_b(t, k, smem + (2 + sb_next) * kSlot);
    return sa_last;
  };
  if (tc.kt > 0) sa = issue(tc, 0, 0);
  bool stored = false;  // previous item ended a tile (8 stores in flight)
  for (;;) {
    if (stored) wait_vmcnt<8>();
    else wait_vmcnt<0>();
    lds_barrier();  // the item's loads are visible; slots of item i-1 are free
    const bool same = ks + 1 < tc.kt;  // false for an empty segment
    int sa_next = sa;
    if (same) sa_next = issue(tc, ks + 1, sb ^ 1);
    else if (tn_ok && tn.kt > 0) sa_next = issue(tn, 0, sb ^ 1);
    if (tc.kt > 0) compute(smem + sa * kSlot, smem + (2 + sb) * kSlot);
    if (!same) {
      lds_barrier();  // every wave is done reading this item's B slot
      epilogue(tc, smem + (2 + sb) * kSlot);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x16_t{};
      if (!tn_ok) break;
      tc = tn;
      ks = 0;
      tn_ok = step();
      if (tn_ok) tn = current();
    } else {
      ++ks;
    }
    stored = !same;
    sa = sa_next;
    sb ^= 1;
  }
}

}  // namespace

extern "C" int moe_grouped_wgrad(const void* at, const uint8_t* at_scales, const void* bt,
                                 const uint8_t* bt_scales, int fmt, const int32_t* kofs, int E,
                                 int M, int N, int64_t kstride, void* dw, hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(E >= 1 && E <= kMaxE && M > 0 && N > 0 && kstride > 0 && kstride % 128 == 0,
              MOE_ERR_INVALID_ARG,
              "moe_grouped_wgrad: need 1 <= E <= 1024, M, N > 0, kstride a positive multiple of 128");
  MOE_REQUIRE(fmt == MOE_MXFP8_E4M3, MOE_ERR_UNSUPPORTED, "moe_grouped_wgrad: fmt must be MXFP8");
  MOE_REQUIRE(M % kTile == 0 && N % kTile == 0, MOE_ERR_INVALID_ARG,
              "moe_grouped_wgrad: need M % 128 == 0 and N % 128 == 0");
  MOE_REQUIRE(at && bt && at_scales && bt_scales && kofs && dw, MOE_ERR_INVALID_ARG,
              "moe_grouped_wgrad: null pointer");
  MOE_REQUIRE(kstride * std::max(M, N) < (int64_t{1} << 32), MOE_ERR_UNSUPPORTED,
              "moe_grouped_wgrad: operand of 4 GiB or more");
  MOE_REQUIRE(aligned16(at) && aligned16(bt) && aligned16(dw) &&
                  (reinterpret_cast<uintptr_t>(at_scales) & 3u) == 0 &&
                  (reinterpret_cast<uintptr_t>(bt_scales) & 3u) == 0,
              MOE_ERR_ALIGNMENT, "moe_grouped_wgrad: tensors must be 16-byte aligned");
  WArgs a;
  a.at = static_cast<const uint8_t*>(at);
  a.at_sc = at_scales;
  a.bt = static_cast<const uint8_t*>(bt);
  a.bt_sc = bt_scales;
  a.kofs = kofs;
  a.E = E;
  a.M = M;
  a.N = N;
  a.dw = static_cast<uint8_t*>(dw);
  a.at_bytes = static_cast<uint32_t>(kstride * M);
  a.at_sc_bytes = static_cast<uint32_t>(kstride / 32 * M);
  a.bt_bytes = static_cast<uint32_t>(kstride * N);
  a.bt_sc_bytes = static_cast<uint32_t>(kstride / 32 * N);
  hipLaunchKernelGGL(wgrad_kernel, dim3(kNumCu * kOcc), dim3(kNT), 0, stream, a);
  return check_launch("grouped wgrad");
}

}  // namespace moe
