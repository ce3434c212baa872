/*
 * moe_mi355x.h — C ABI of a sigmoid-routed mixture-of-experts layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer is the routed MoE of the page "[PyTorch] DeepSeekV3Layer: full
 * MoE transformer layer (MLA + DeepSeek MoE)" (TransformerEngine pull
 * request), section Description, DeepSeekV3MoE item: a fused sigmoid router
 * with an aux-loss-free (selection-only) bias and grouped top-k, experts
 * built as GroupedLinear -> ScaledSwiGLU -> GroupedLinear, local routing,
 * and an optional shared expert. Its Performance section ("Where the time
 * goes" table) names the remaining steps: a local permute into an
 * expert-major staging buffer with zero-filled padding, the fused grouped
 * MLP (fc1+SwiGLU, fc2, dGLU backward, wgrad) and MXFP8 quantization of the
 * received rows. The 4-bit W4A4 MoE of "Mistral Large 3 NVFP4 TRTLLM MoE
 * support" (sglang pull request, Modifications section) is served here by
 * MXFP4.
 *
 * A forward pass is:
 *   moe_route -> [moe_quantize_mx] -> moe_permute -> moe_grouped_mlp_fwd
 *   (routed experts; again with E = 1 for a shared expert) -> moe_combine
 * where moe_grouped_mlp_fwd is moe_grouped_fc1_swiglu followed by
 * moe_grouped_fc2 (moe_grouped_fc1_swiglu_dense / moe_grouped_fc2_dense run
 * the routed and the shared expert in the same launches). The backward of
 * the routed experts is moe_grouped_mlp_bwd.
 *
 * Conventions for every call
 *   - Pointers are device pointers owned by the caller unless stated; the
 *     library never allocates and keeps no state between calls. Scratch
 *     memory comes from the caller (size queries *_workspace); the one
 *     exception, moe_permute_noalloc, uses a fixed array of its own.
 *   - Tensors are dense and row-major; pointers to tensors must be 16-byte
 *     aligned, and row strides are whole rows (no padding between rows).
 *   - MX tensors: element codes [rows, K] bytes (E4M3) or [rows, K/2] bytes
 *     (E2M1, two per byte, the even element in the low nibble), plus E8M0
 *     scale bytes [rows, K/32] (scale = 2^(byte - 127)); blocks of 32
 *     consecutive elements along K share one scale. K % 32 == 0.
 *   - Calls are asynchronous on `stream` (0 = the null stream). All argument
 *     checks run on the host before anything is enqueued: a call that
 *     returns an error has enqueued nothing. Device faults surface at the
 *     caller's next synchronization.
 *   - Every call returns MOE_OK (0) or a negative moe_status;
 *     moe_last_error() returns a message for the calling thread's last
 *     failure. No C++ exception crosses the ABI.
 *   - Calls touch only their arguments, so concurrent calls on different
 *     streams with disjoint outputs are safe.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,  /* bad shape, bad enum value or null pointer  */
  MOE_ERR_UNSUPPORTED = -2,  /* valid but unsupported format combination   */
  MOE_ERR_ALIGNMENT = -3,    /* pointer or row size not 16-byte aligned    */
  MOE_ERR_WORKSPACE = -4,    /* workspace missing or too small             */
  MOE_ERR_HIP = -5           /* the HIP runtime reported a launch error    */
} moe_status;

typedef enum moe_format {
  MOE_F32 = 0,               /* IEEE binary32                              */
  MOE_BF16 = 1,              /* bfloat16                                   */
  MOE_MXFP8_E4M3 = 2,        /* E4M3 codes + E8M0 scales per 32 along K    */
  MOE_MXFP4_E2M1 = 3,        /* E2M1 codes (packed) + E8M0 scales per 32   */
  MOE_NVFP4_E2M1 = 4         /* E2M1 codes (packed) + E4M3 scales per 16
                                + one fp32 scale per tensor               */
} moe_format;

/* Version of this ABI (MOE_ABI_VERSION of the built library). */
int moe_abi_version(void);

/* Static text for a status code. */
const char* moe_status_str(int status);

/* Message of the calling thread's most recent failed call ("" if none). */
const char* moe_last_error(void);

/*
 * moe_route — router GEMM, sigmoid scores, selection bias, grouped top-k,
 * normalized and scaled combine weights. (TE DeepSeekV3Layer page,
 * Description, DeepSeekV3MoE item: "fused sigmoid router with aux-loss-free
 * bias and grouped top-k".)
 *
 *   logits[t, e] = sum_h x[t, h] * w_router[e, h]      (fp32 accumulate)
 *   s = sigmoid(logits) evaluated in fp64, rounded once to fp32
 *   sel = fp32(s + bias)                               (selection only)
 *   n_group > 1: experts form n_group contiguous groups; a group scores the
 *     fp32 sum of its two largest sel values; the topk_group best groups are
 *     kept (ties: lower group index), all other experts are excluded
 *   topk_idx[t, 0..k-1]: the k largest remaining sel, descending (ties:
 *     lower expert index)
 *   topk_w[t, j] = fp32(fp32(s[idx] / S) * routed_scale), S the fp32 sum of
 *     the k chosen s in slot order
 *
 * x          [T, H] in x_fmt (MOE_F32 or MOE_BF16); w_router [E, H] in the
 *            same format. Both may be NULL when logits_in is given.
 * bias       [E] fp32 selection bias (required).
 * logits_in  optional [T, E] fp32: when non-NULL the GEMM is skipped and
 *            selection starts from these logits.
 * logits_out optional [T, E] fp32: receives the logits used.
 * topk_idx   [T, k] int32 out; topk_w [T, k] fp32 out.
 * ws         device workspace of at least moe_route_workspace(T, H, E)
 *            bytes for the router GEMM's partial sums (the GEMM is split
 *            along H when T is small; the partials are added in a fixed
 *            order); may be NULL when logits_in is given. Otherwise
 *            MOE_ERR_WORKSPACE.
 * Limits: 1 <= E <= 512, E % n_group == 0, E / n_group >= 2 when
 * n_group > 1, 1 <= topk_group <= n_group, 1 <= k <= min(16,
 * topk_group * E / n_group), H % 32 == 0 (bf16) when the GEMM runs.
 * T == 0 is a no-op (after the checks of E, n_group, topk_group and k; the
 * pointers may then be NULL).
 */
int moe_route(const void* x, int x_fmt, const void* w_router, const float* bias,
              const float* logits_in, int T, int H, int E, int n_group,
              int topk_group, int k, float routed_scale, float* logits_out,
              int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
              hipStream_t stream);

/* moe_route_workspace — bytes of moe_route's workspace (0 for bad sizes). */
size_t moe_route_workspace(int T, int H, int E);

/*
 * moe_quantize_mx — MX block quantization of a [rows, K] tensor along K
 * (TE DeepSeekV3Layer page, Performance section, "Where the time goes":
 * MXFP8 quantization of the received rows and of dense GEMM inputs).
 *
 * Per row and per block of 32 consecutive elements v along K:
 *   amax = max |v|; amax == 0 -> scale byte 0;
 *   otherwise e = floor(log2 amax) - emax (emax 8 for E4M3, 2 for E2M1),
 *   clamped to [-127, 127], scale byte = e + 127;
 *   code = element-grid value nearest to v / 2^e, ties to the even code,
 *   saturated to +-448 (E4M3) / +-6 (E2M1); the code keeps v's sign bit.
 * in      [rows, K] in in_fmt (MOE_F32 or MOE_BF16); rows may be 0.
 * out_fmt MOE_MXFP8_E4M3 or MOE_MXFP4_E2M1.
 * axis 0  blocks of 32 along K: codes [rows, K] (E4M3) or [rows, K/2]
 *         (E2M1), scales [rows, K/32].
 * axis 1  blocks of 32 consecutive rows of each column, output K-major
 *         (transposed): codes [K, rows] or [K, rows/2], scales [K, rows/32];
 *         needs in_fmt MOE_BF16 and rows % 32 == 0. This is the layout a
 *         GEMM contracting over the rows consumes (the backward's
 *         transposed weight copies).
 */
int moe_quantize_mx(const void* in, int in_fmt, int64_t rows, int K, int axis,
                    int out_fmt, uint8_t* codes, uint8_t* scales,
                    hipStream_t stream);

/*
 * moe_permute_rows_bound — rows of the expert-major buffer:
 * T*k + E*(align-1). Returns -1 for invalid arguments.
 */
int64_t moe_permute_rows_bound(int T, int k, int E, int align);

/* moe_permute_workspace — scratch bytes moe_permute needs. */
size_t moe_permute_workspace(int T, int k, int E);

/*
 * moe_permute — expert-major permutation (TE DeepSeekV3Layer page,
 * Performance section, "Where the time goes": local permute "dup" into an
 * expert-major staging buffer with zero-filled padding).
 *
 *   counts[e]   number of (t, j) with topk_idx[t, j] == e
 *   offsets[e]  sum over e' < e of counts[e'] rounded up to `align`;
 *               offsets[E] is the used row count
 *   row_map[t, j]  offsets[e] + rank of (t, j) among the pairs of expert e
 *               in (t, j) lexicographic order (a stable order)
 *   src_row[r]  token of row r, or -1 for every padding row, for all
 *               r < moe_permute_rows_bound(T, k, E, align)
 *   rows_out[r] = rows_in[src_row[r]] (row_bytes opaque bytes), zero bytes
 *               for padding rows; scales_out likewise with scale_bytes per
 *               row (for MX rows). Zero bytes decode to 0 in every format.
 * Built with a per-wave histogram, a column scan and a stable scatter; no
 * atomics, so results are deterministic.
 *
 * topk_idx [T, k] int32 with values in [0, E) (values outside give
 *          undefined maps; not checked on the device).
 * rows_in / rows_out: optional (both NULL: maps only). row_bytes % 16 == 0.
 * scales_in / scales_out: optional, scale_bytes > 0 when given.
 * align in {1, 16, 32, 64, 128}. ws: moe_permute_workspace(T, k, E) bytes.
 * counts [E], offsets [E+1], row_map [T, k], src_row [bound] int32 out.
 */
int moe_permute(const int32_t* topk_idx, int T, int k, int E, int align,
                const void* rows_in, int64_t row_bytes, const void* scales_in,
                int64_t scale_bytes, int32_t* counts, int32_t* offsets,
                int32_t* row_map, int32_t* src_row, void* rows_out,
                void* scales_out, void* ws, size_t ws_bytes,
                hipStream_t stream);

/*
 * moe_permute_noalloc — moe_permute for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments, results and checks as moe_permute,
 * without ws / ws_bytes: the histogram lives in a fixed 1 MiB array inside
 * the library (one copy per GPU, held until the process ends, its device
 * address looked up once per device on the first call there). The call
 * allocates nothing.
 * Limit: moe_permute_workspace(T, k, E) <= moe_permute_noalloc_max_bytes()
 * (1 MiB: ceil(T * k / 1024) * E * 4 bytes), else MOE_ERR_WORKSPACE with
 * nothing enqueued. The array keeps the last call's contents (the first
 * kernel rewrites every entry it later reads, so nothing needs clearing).
 * Calls that overlap on one GPU (different streams or threads) share the
 * array and race: serialize them.
 */
int moe_permute_noalloc(const int32_t* topk_idx, int T, int k, int E, int align,
                        const void* rows_in, int64_t row_bytes,
                        const void* scales_in, int64_t scale_bytes,
                        int32_t* counts, int32_t* offsets, int32_t* row_map,
                        int32_t* src_row, void* rows_out, void* scales_out,
                        hipStream_t stream);

/* moe_permute_noalloc_max_bytes — size of moe_permute_noalloc's fixed
 * histogram array (the largest moe_permute_workspace it accepts). */
size_t moe_permute_noalloc_max_bytes(void);

/*
 * moe_grouped_mlp_workspace — scratch bytes of moe_grouped_mlp_fwd (the
 * SwiGLU output h of every row, plus its MX scales for MX formats).
 */
size_t moe_grouped_mlp_workspace(int E, int H, int F, int64_t rows, int a_fmt,
                                 int w_fmt);

/*
 * moe_pack_weights — one-time preparation of expert weights for the grouped
 * GEMMs (done when the weights change, not per step): reorders each
 * expert's [N, K] matrix so that a wavefront streams exactly the bytes its
 * 32x32 matrix instructions consume, contiguously. (TE DeepSeekV3Layer
 * page, Description and Performance section: the experts' GroupedLinear
 * weights of the fused grouped MLP; MX scales one per 32 values along K.)
 * Layout: for expert e, 32-row column block cb, 128-byte K stage s, piece
 * q < 4 and lane l < 64, 16 bytes = bytes [128 s + 32 q + 16 (l / 32), +16)
 * of row R(cb, l): R = 32 cb + l % 32, or with half = F > 0 (fc1, N = 2F)
 * gate row 32 (cb / 2) + l % 32 for even cb and up row F + 32 (cb / 2) +
 * l % 32 for odd cb. MX scales: for (e, cb, s, l), kSub bytes (2 for
 * E4M3, 4 for E2M1): byte j is the scale of stage-local 32-block
 * 2 j + l / 32 of row R(cb, l).
 * w        [E, N, K] in fmt (BF16 values, or MX codes with w_scales
 *          [E, N, K/32]); out (and out_scales) the same number of bytes.
 * NVFP4 (fmt MOE_NVFP4_E2M1; codes [E, N, K/2], w_scales [E, N, K/16] as
 * moe_quantize_nvfp4 writes them): 64-value stages s; for (e, cb, s, l)
 * 16 bytes = for k-step j < 4 the 4 code bytes at byte 32 s + 8 j +
 * 4 (l / 32) of row R(cb, l); scales for (e, cb, s, r < 32) 4 bytes = the
 * E4M3 scales of row R(cb, r)'s 16-blocks 4 s + j (both lane halves read
 * the same word).
 * Limits: N % 64 == 0; K a multiple of 64 (BF16, NVFP4), 128 (E4M3), 256
 * (E2M1); half == 0 or N == 2 * half with half % 32 == 0.
 */
int moe_pack_weights(const void* w, const uint8_t* w_scales, int fmt, int E,
                     int N, int K, int half, void* out, uint8_t* out_scales,
                     hipStream_t stream);

/*
 * moe_grouped_mlp_fwd — per expert e, on rows [offsets[e], offsets[e+1]):
 *   A = X_e . W1_e^T          [n_e, 2F], fp32 accumulate
 *   h = silu(A[:, :F]) * A[:, F:]   (W1 rows [0, F) gate, [F, 2F) up)
 *   (MX formats: h is MX-quantized per row along F before fc2)
 *   y = h . W2_e^T            [n_e, H]
 * (TE DeepSeekV3Layer page, Description: GroupedLinear -> ScaledSwiGLU ->
 * GroupedLinear; the routing weight is applied later by moe_combine, which
 * equals scaling h since fc2 has no bias. sglang page, Highlights: fc1's
 * weight holds the w1 (gate) and w3 (up) halves.)
 *
 * a        activations: [rows, H] in a_fmt (MOE_F32, MOE_BF16, or MX codes)
 *          indexed by row, or — when src_row is non-NULL — token rows
 *          [T, H] gathered through src_row (row r reads a[src_row[r]]; a
 *          row with src_row -1 produces zero h).
 * a_scales MX scales of a ([rows or T, H/32]), NULL for F32/BF16.
 * w1       [E, 2F, H] and w2 [E, H, F] in w_fmt: for BF16 and MX formats
 *          packed by moe_pack_weights (w1 with half = F, w2 with half = 0),
 *          with their packed MX scales w1_scales / w2_scales (NULL for BF16);
 *          for F32 plain row-major, no scales.
 * Supported (a_fmt, w_fmt, y_fmt): (F32, F32, F32), (BF16, BF16, BF16),
 *          (MXFP8, MXFP8, BF16), (MXFP4, MXFP4, BF16).
 * offsets  [E+1] int32 device array (as moe_permute writes it);
 *          offsets[E] <= rows.
 * act_save optional [rows, 2F] fp32: receives A = (gate | up) unrounded,
 *          for the backward (rows of a padding slot hold unspecified values).
 * y        [rows, H] in y_fmt; rows outside every segment are not written.
 * ws       moe_grouped_mlp_workspace(E, H, F, rows, a_fmt, w_fmt) bytes.
 * Limits: 1 <= E <= 1024; BF16: H % 128 == 0, F % 64 == 0; MXFP8:
 * H % 128 == 0, F % 128 == 0; MXFP4: H % 256 == 0, F % 256 == 0.
 * A shared expert is a call with E = 1, offsets = {0, T} and src_row NULL.
 */
int moe_grouped_mlp_fwd(const void* a, const uint8_t* a_scales, int a_fmt,
                        const int32_t* src_row, const void* w1,
                        const uint8_t* w1_scales, const void* w2,
                        const uint8_t* w2_scales, int w_fmt,
                        const int32_t* offsets, int E, int H, int F,
                        int64_t rows, float* act_save, void* y, int y_fmt,
                        void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_grouped_fc1_swiglu — the first half of moe_grouped_mlp_fwd on its
 * own: per expert segment, A = X_e . W1_e^T and h = silu(A[:, :F]) * A[:, F:]
 * (MX formats: h MX-quantized per row along F). Same argument meaning,
 * formats and limits as moe_grouped_mlp_fwd; w_fmt must equal a_fmt.
 * h        [rows, F] out in a_fmt (F32, BF16, or MX codes [rows, F] /
 *          [rows, F/2]); h_scales [rows, F/32] out for MX (NULL otherwise).
 *          Rows outside every segment are not written.
 * rows == 0 is a no-op after the checks of E, H, F and the formats; the
 * pointers may then be NULL.
 */
int moe_grouped_fc1_swiglu(const void* a, const uint8_t* a_scales, int a_fmt,
                           const int32_t* src_row, const void* w1,
                           const uint8_t* w1_scales, int w_fmt,
                           const int32_t* offsets, int E, int H, int F,
                           int64_t rows, float* act_save, void* h,
                           uint8_t* h_scales, hipStream_t stream);

/*
 * moe_grouped_fc2 — the second half: per expert segment y = h_e . W2_e^T.
 * h        [rows, F] in h_fmt with h_scales for MX (as fc1 writes them).
 * w2       [E, H, F] in w_fmt (== h_fmt) with w2_scales [E, H, F/32] for MX.
 * y        [rows, H] in y_fmt (F32 for the F32 layer, BF16 otherwise).
 * rows == 0 is a no-op after the same checks; the pointers may then be NULL.
 */
int moe_grouped_fc2(const void* h, const uint8_t* h_scales, int h_fmt,
                    const void* w2, const uint8_t* w2_scales, int w_fmt,
                    const int32_t* offsets, int E, int H, int F, int64_t rows,
                    void* y, int y_fmt, hipStream_t stream);

/*
 * moe_grouped_fc1_swiglu_dense / moe_grouped_fc2_dense — the routed grouped
 * fc1 (resp. fc2) and the layer's always-on shared expert (TE DeepSeekV3Layer
 * page, Description: optional shared expert) in one launch. The shared
 * expert takes all T token rows and has the routed experts' format and
 * shape (F_shared == F); its weights w1d [2F, H] (gate rows then up rows) /
 * w2d [H, F], packed by moe_pack_weights like one routed expert (w1d with
 * half = F). Arguments as moe_grouped_fc1_swiglu / moe_grouped_fc2, except:
 * fc1: h (+ h_scales) has rows + T rows; row rows + t holds the shared
 *      expert's h of token t, computed from row t of `a` (no gather);
 *      act_save covers the routed rows only.
 * fc2: h and y have rows + T rows; rows [rows, rows + T) are the shared
 *      expert's input and output.
 * Not for fp32 layers (MOE_ERR_UNSUPPORTED). The shared expert's tiles are
 * spread through the routed experts' tile list.
 */
int moe_grouped_fc1_swiglu_dense(const void* a, const uint8_t* a_scales, int a_fmt,
                                 const int32_t* src_row, const void* w1,
                                 const uint8_t* w1_scales, int w_fmt,
                                 const int32_t* offsets, int E, int H, int F,
                                 int64_t rows, float* act_save, void* h,
                                 uint8_t* h_scales, const void* w1d,
                                 const uint8_t* w1d_scales, int T, hipStream_t stream);
int moe_grouped_fc2_dense(const void* h, const uint8_t* h_scales, int h_fmt,
                          const void* w2, const uint8_t* w2_scales, int w_fmt,
                          const int32_t* offsets, int E, int H, int F, int64_t rows,
                          void* y, int y_fmt, const void* w2d,
                          const uint8_t* w2d_scales, int T, hipStream_t stream);

/*
 * NVFP4 W4A4 expert MLP (sglang "Mistral Large 3 NVFP4 TRTLLM MoE support"
 * page, title and Modifications: W4A4 NVFP4 MoE). Format: E2M1 codes two per
 * byte (even element low nibble), one E4M3 scale per 16 consecutive values
 * along K, one fp32 scale g per tensor; value = e2m1 * e4m3 * g. The block
 * rule: s = E4M3 RNE(min(amax16 / fp32(6 g), 448)), codes = E2M1 RNE of
 * clamp(v / fp32(s g), -6, 6) with v's sign bit (zero codes when s is 0).
 * A weight matrix's g = amax / 2688 (1 for an all-zero matrix); the
 * activations of a layer take fixed scales (x_g, h_g) from the caller.
 */

/*
 * moe_nvfp4_tensor_scale — g[i] = fp32(amax(tensor i) / 2688), or 1 when
 * tensor i is all zero, for n_tensors consecutive tensors of
 * elems_per_tensor elements each of `in` (MOE_BF16 or MOE_F32, device).
 * g: [n_tensors] fp32 device (its bytes are used as scratch first).
 */
int moe_nvfp4_tensor_scale(const void* in, int in_fmt, int n_tensors,
                           int64_t elems_per_tensor, float* g, hipStream_t stream);

/*
 * moe_quantize_nvfp4 — NVFP4 block quantization of [rows, K] (MOE_BF16 or
 * MOE_F32, row-major, device) along K; row r uses the tensor scale
 * g[r / rows_per_tensor]. Outputs (each optional, at least one given):
 * codes [rows, K/2] packed E2M1 (8-byte aligned), scales [rows, K/16] E4M3,
 * vals [rows, K] bf16 = e2m1 * e4m3 (exact; the operand the NVFP4 GEMMs
 * take for activations, the tensor scale left out). K % 16 == 0. The
 * codes depend only on the input bits and g (IEEE fp32 divisions).
 */
int moe_quantize_nvfp4(const void* in, int in_fmt, int64_t rows, int K,
                       int64_t rows_per_tensor, const float* g, uint8_t* codes,
                       uint8_t* scales, void* vals, hipStream_t stream);

/*
 * moe_grouped_fc1_swiglu_nvfp4 — per expert segment (as
 * moe_grouped_fc1_swiglu), with NVFP4 activations and weights:
 *   A = x_g * w1_g[e] * (Xv_e . W1v_e^T)   (fp32 accumulate of exact products)
 *   h = silu(A[:, :F]) * A[:, F:], NVFP4-quantized along F with scale h_g.
 * a_vals   [rows or T, H] bf16 operand values of x (moe_quantize_nvfp4's
 *          vals with tensor scale x_g), gathered through src_row as in
 *          moe_grouped_fc1_swiglu when src_row is non-NULL.
 * w1, w1_scales  NVFP4 [E, 2F, H] packed by moe_pack_weights (half = F);
 *          w1_g [E] fp32 device: each expert matrix's tensor scale.
 * h_vals   [rows, F] bf16 out: operand values of h (code * scale, h's
 *          tensor scale h_g left out). Rows outside every segment are not
 *          written.
 * Limits: 1 <= E <= 1024, H % 128 == 0, F % 64 == 0; x_g, h_g > 0.
 */
int moe_grouped_fc1_swiglu_nvfp4(const void* a_vals, const int32_t* src_row,
                                 const void* w1, const uint8_t* w1_scales,
                                 const float* w1_g, float x_g, float h_g,
                                 const int32_t* offsets, int E, int H, int F,
                                 int64_t rows, void* h_vals, hipStream_t stream);

/*
 * moe_grouped_fc2_nvfp4 — per expert segment y = h_g * w2_g[e] *
 * (Hv_e . W2v_e^T) in bf16 [rows, H]; h_vals as fc1 writes them, w2 /
 * w2_scales NVFP4 [E, H, F] packed by moe_pack_weights (half = 0), w2_g
 * [E] fp32 device. Same limits as the fc1 entry.
 */
int moe_grouped_fc2_nvfp4(const void* h_vals, const void* w2, const uint8_t* w2_scales,
                          const float* w2_g, float h_g, const int32_t* offsets, int E,
                          int H, int F, int64_t rows, void* y, hipStream_t stream);

/*
 * moe_combine — weighted top-k reduce back to token order (TE
 * DeepSeekV3Layer page, Performance section, "Where the time goes": local
 * permute "reduce"; Description: optional shared expert added).
 *   out[t] = sum_{j<k} topk_w[t, j] * y[row_map[t, j]]  (+ shared[t])
 * accumulated in fp32 in slot order j = 0..k-1.
 * y [rows, H] in y_fmt (MOE_F32 or MOE_BF16); shared optional [T, H] in
 * y_fmt; out [T, H] in out_fmt (MOE_F32 or MOE_BF16). H % 8 == 0, k <= 16.
 */
int moe_combine(const void* y, int y_fmt, const int32_t* row_map,
                const float* topk_w, const void* shared, int T, int k, int H,
                void* out, int out_fmt, hipStream_t stream);

/*
 * ---- Backward of the routed expert path (TE DeepSeekV3Layer page,
 * Performance section, "Where the time goes": dGLU bwd and wgrad of the
 * fused grouped MLP in MXFP8; the local permute's reduce). Routing weights
 * are constants and quantizers pass gradients straight through.
 * moe_grouped_mlp_bwd (at the end of this header) runs the whole backward
 * in one call; its steps are also exported one by one, in this order:
 *   moe_combine_bwd (dY rows, MX) -> moe_grouped_fc2_dgrad_dswiglu ->
 *   moe_grouped_fc1_dgrad -> moe_unpermute ->
 *   moe_quantize_mx_segments (dY, h, dA, x) -> moe_grouped_wgrad (dW2, dW1)
 */

/*
 * moe_combine_bwd — dY rows of the expert-major layout:
 *   dy[r] = topk_w[t, j] * dout[t]   for r = row_map[t, j]
 * formed in fp32; every row with src_row[r] == -1 is zero.
 * dout    [T, H] in dout_fmt (MOE_BF16 or MOE_F32).
 * dy      [rows, H] out in dy_fmt: MOE_F32, MOE_BF16, or an MX format (codes
 *         [rows, H] / [rows, H/2] encoded from the fp32 products, with
 *         dy_scales [rows, H/32]; needs H % 32 == 0).
 * row_w   optional [rows] fp32 out: the routing weight of each row (0 for a
 *         padding row), the row scale moe_quantize_mx_segments takes to form
 *         the same dY rows from dout.
 */
int moe_combine_bwd(const void* dout, int dout_fmt, const int32_t* row_map,
                    const int32_t* src_row, const float* topk_w, int T, int k,
                    int H, int64_t rows, void* dy, int dy_fmt,
                    uint8_t* dy_scales, float* row_w, hipStream_t stream);

/*
 * moe_unpermute — dx[t] = sum_j dx_perm[row_map[t, j]], fp32 accumulation
 * in slot order (the permute "reduce" of the backward). With k = 1 it is
 * the exact inverse of moe_permute's gather.
 * dx_perm [rows, H] and dx [T, H] in MOE_F32 or MOE_BF16.
 */
int moe_unpermute(const void* dx_perm, int fmt, const int32_t* row_map, int T,
                  int k, int H, void* dx, int out_fmt, hipStream_t stream);

/* moe_segments_kstride — row width (elements) of the K-major outputs of
 * moe_quantize_mx_segments: rows + 127*E rounded up to 128. -1 if invalid. */
int64_t moe_segments_kstride(int64_t rows, int E);

/*
 * moe_quantize_mx_segments — MX quantization of expert-major rows along the
 * rows of each expert segment (the weight-gradient operands): segment e is
 * rows [offsets[e], offsets[e+1]) (lengths multiples of 32, as moe_permute
 * with align 32 writes them); channel c of segment e becomes the K values
 * kofs[e] .. kofs[e] + len_e in blocks of 32 rows, the segment padded with
 * zeros to a multiple of 128, kofs[e] the sum of the padded lengths before
 * e (written to kofs [E+1]). Values are formed in fp32:
 * mode 0: in [rows, C], row r used as is (zero where src_row[r] < 0)
 * mode 1: in [T, C] token rows gathered through src_row (zero for -1)
 * mode 2: in [rows, 2C] = the saved fc1 output (gate | up); the value
 *         is silu(gate) * up (h recomputed), zero where src_row[r] < 0
 * in_fmt  MOE_BF16 or MOE_F32.
 * row_scale optional [rows] fp32: row r's values are multiplied by
 *         row_scale[r] (mode 1 with moe_combine_bwd's row_w gives dY).
 * out_fmt MOE_MXFP8_E4M3. Stage-major layout: K is cut into stages of 128;
 * codes [kstride/128][C][128]: stage g, channel c holds the E4M3 codes of K
 * values [128g, 128g + 128) (one 128-channel block of a stage is 16 KB
 * contiguous); scales [kstride/128][C][4], byte j the E8M0 scale of K block
 * [128g + 32j, +32). kstride >= moe_segments_kstride(rows, E), a multiple
 * of 128; stages past kofs[E] / 128 are not written. C % 8 == 0; in and
 * codes 16-byte aligned, scales 4-byte aligned.
 */
int moe_quantize_mx_segments(const void* in, int in_fmt, int mode,
                             const int32_t* src_row, const int32_t* offsets,
                             const float* row_scale, int E, int64_t rows,
                             int C, int64_t kstride, int out_fmt,
                             uint8_t* codes, uint8_t* scales, int32_t* kofs,
                             hipStream_t stream);

/*
 * moe_grouped_fc2_dgrad_dswiglu — per expert segment, dH = dY . W2 with W2
 * given transposed w2t [E, F, H] (contraction over H contiguous, packed by
 * moe_pack_weights with half = 0, scales packed alongside), then the
 * SwiGLU backward with the saved fc1 output A = (g | u):
 *   dgate = dH * u * sig(g) * (1 + g * (1 - sig(g))),  dup = dH * silu(g)
 * dy      [rows, H] in fmt (MX: codes + dy_scales [rows, H/32]).
 * act_save [rows, 2F] fp32 (moe_grouped_fc1_swiglu's act_save).
 * da      [rows, 2F] out: MX codes (+ da_scales [rows, 2F/32], blocks along
 *         2F) or bf16 when fmt is MOE_BF16; da_f32 optional fp32 copy of the
 *         unrounded dA (the weight gradient's operand).
 * Limits: H % 128 == 0 (256 for MXFP4), F % 128 == 0.
 */
int moe_grouped_fc2_dgrad_dswiglu(const void* dy, const uint8_t* dy_scales,
                                  int fmt, const void* w2t,
                                  const uint8_t* w2t_scales,
                                  const int32_t* offsets, int E, int H, int F,
                                  int64_t rows, const float* act_save, void* da,
                                  uint8_t* da_scales, float* da_f32,
                                  hipStream_t stream);

/*
 * moe_grouped_fc1_dgrad — per expert segment dX_rows = dA . W1 with W1 given
 * transposed w1t [E, H, 2F] (contraction over 2F contiguous, packed by
 * moe_pack_weights with half = 0).
 * da [rows, 2F] in fmt (MX codes + da_scales); dx_perm [rows, H] bf16 out.
 */
int moe_grouped_fc1_dgrad(const void* da, const uint8_t* da_scales, int fmt,
                          const void* w1t, const uint8_t* w1t_scales,
                          const int32_t* offsets, int E, int H, int F,
                          int64_t rows, void* dx_perm, hipStream_t stream);

/*
 * moe_grouped_wgrad — per expert e, dw[e] = A_e^T-contracted product over
 * the K segment [kofs[e], kofs[e+1]):  dw[e][m, n] = sum_k at[m, k] bt[n, k]
 * at (M channels) and bt (N channels): MXFP8 codes and scales in the
 * stage-major layout of moe_quantize_mx_segments (codes [kstride/128][M or
 * N][128], scales [kstride/128][M or N][4]); kofs as that call writes it
 * (kofs[E] <= kstride); dw [E, M, N] bf16 out; an expert with an empty
 * segment gets exact zeros.
 * Limits: fmt MOE_MXFP8_E4M3; M % 128 == 0, N % 128 == 0; kstride % 128 == 0;
 * kofs[e] multiples of 128 (as moe_quantize_mx_segments writes them).
 */
int moe_grouped_wgrad(const void* at, const uint8_t* at_scales, const void* bt,
                      const uint8_t* bt_scales, int fmt, const int32_t* kofs,
                      int E, int M, int N, int64_t kstride, void* dw,
                      hipStream_t stream);

/*
 * moe_grouped_mlp_bwd_workspace — scratch bytes of moe_grouped_mlp_bwd (0
 * for unsupported arguments).
 */
size_t moe_grouped_mlp_bwd_workspace(int T, int k, int E, int H, int F,
                                     int64_t rows, int fmt);

/*
 * moe_grouped_mlp_bwd — the whole backward of the routed expert path in one
 * call (TE DeepSeekV3Layer page, Performance section, "Where the time
 * goes": the fused grouped MLP's dGLU bwd and wgrad in MXFP8, the local
 * permute's reduce). Routing weights are constants; quantizers pass
 * gradients straight through. On `stream` it runs, in order:
 *   dY rows = topk_w[t, j] * dout[t] (fp32, MX-encoded along H)
 *   dH = dY . W2, dA = SwiGLU'(dH; A) with A = act_save (dA in MX along 2F
 *     and in fp32)
 *   dX rows = dA . W1 (bf16); dx[t] = sum_j dX rows[row_map[t, j]] (fp32 in
 *     slot order, rounded to act_fmt)
 *   dw2[e] = dY_e^T . h_e, dw1[e] = dA_e^T . x_e over the rows of each
 *     expert segment, operands MX-quantized along those rows in blocks of 32
 *     (dY formed again from dout and the routing weights, h recomputed from
 *     act_save); an expert with no rows gets exact zeros.
 * dout, x   [T, H] in act_fmt (MOE_BF16 or MOE_F32); dx [T, H] out in act_fmt.
 * row_map [T, k], src_row [rows], offsets [E+1] (moe_permute's maps with
 *          align 32, so every segment is a whole number of 32-row blocks),
 *          topk_w [T, k] fp32 (moe_route's weights).
 * act_save [rows, 2F] fp32: the forward's fc1 output (gate | up).
 * w1t [E, H, 2F] and w2t [E, F, H]: the transposed weight copies, MX-
 *          quantized along their contraction axis and packed by
 *          moe_pack_weights (half = 0), with their packed scales.
 * dw1 [E, 2F, H], dw2 [E, H, F] bf16 out.
 * ws       moe_grouped_mlp_bwd_workspace(T, k, E, H, F, rows, fmt) bytes,
 *          16-byte aligned.
 * Limits: fmt MOE_MXFP8_E4M3; H % 128 == 0, F % 128 == 0, 1 <= E <= 1024,
 * 1 <= k <= 16, T * k <= rows < 2^31. All checks run before the first
 * kernel is enqueued. With T == 0, dout, x, row_map, topk_w and dx may be
 * NULL (dw1 and dw2 are still written: all zeros).
 */
int moe_grouped_mlp_bwd(const void* dout, const void* x, int act_fmt,
                        const int32_t* row_map, const int32_t* src_row,
                        const float* topk_w, const int32_t* offsets,
                        const float* act_save, const void* w1t,
                        const uint8_t* w1t_scales, const void* w2t,
                        const uint8_t* w2t_scales, int fmt, int T, int k, int E,
                        int H, int F, int64_t rows, void* dx, void* dw1,
                        void* dw2, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * ---- Training steps around the routing (TE DeepSeekV3Layer page,
 * Description, DeepSeekV3MoE item: sigmoid router with an aux-loss-free
 * bias and grouped top-k; Changes section: optional sequence-wise aux
 * loss). The pages give no formula; these are the DeepSeek-V3 rules.
 */

/* moe_route_bwd_workspace — scratch bytes of moe_route_bwd (0 if invalid;
 * seq_len 0 when the balance loss is off). */
size_t moe_route_bwd_workspace(int T, int H, int E, int seq_len);

/*
 * moe_route_bwd — the router backward of one layer pass. The expert lists
 * are constants and the bias takes no gradient (it only selects):
 *   dw[t, j]   = <dout[t], y[row_map[t, j]]>   (fp32)
 *   ds[t, e_j] = routed_scale / S_t * (dw[t, j] - sum_i dw[t, i] s[t, e_i] / S_t),
 *                s = sigmoid(logits), S_t = sum_j s[t, e_j]; 0 off the list
 *   dlogits    = ds * s * (1 - s)
 *                + (aux_alpha != 0) the sequence-wise balance-loss gradient:
 *                loss = aux_alpha * mean over sequences of L = seq_len
 *                consecutive tokens of sum_i f_i P_i, f_i = E / (k L) *
 *                (tokens of the sequence selecting i), P_i = mean over the
 *                sequence of s[t, i] / sum_m s[t, m]
 *   dx_router  = dlogits . w_router   [T, H] bf16
 *   dw_router  = dlogits^T . x        [E, H] fp32
 * The two products run on bf16 matrix cores with dlogits rounded to bf16
 * (fp32 accumulation).
 * dout [T, H], x [T, H], w_router [E, H], y [rows, H] (the forward's expert
 *          output rows, before weighting) in act_fmt = MOE_BF16.
 * row_map, topk_idx [T, k] int32 and logits [T, E] fp32: the forward's.
 * dlogits optional [T, E] fp32 out; aux_loss [1] fp32 out (required when
 *          aux_alpha != 0).
 * Limits: E a multiple of 8 in [8, 512], 1 <= k <= min(16, E), H % 8 == 0,
 * seq_len dividing T when aux_alpha != 0. T == 0 is a no-op.
 */
int moe_route_bwd(const void* dout, const void* y, int act_fmt,
                  const int32_t* row_map, const int32_t* topk_idx,
                  const float* logits, const void* x, const void* w_router, int T,
                  int k, int E, int H, float routed_scale, int seq_len,
                  float aux_alpha, float* dlogits, float* aux_loss,
                  void* dx_router, float* dw_router, void* ws, size_t ws_bytes,
                  hipStream_t stream);

/*
 * moe_bias_update — the aux-loss-free bias update after a step:
 *   bias_out[e] = bias[e] + gamma * sign(T k / E - counts[e])
 * with counts the per-expert loads moe_permute wrote (T k their sum); the
 * sign is taken exactly in integers, the sum is one fp32 addition.
 * bias_out may equal bias. 1 <= E <= 1024.
 */
int moe_bias_update(const int32_t* counts, int E, float gamma, const float* bias,
                    float* bias_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
