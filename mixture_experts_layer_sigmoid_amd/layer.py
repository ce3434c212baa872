"""One forward pass of the routed MoE layer as a sequence of C-ABI calls.

The object preallocates every buffer the pass needs (torch device memory)
and then issues, on one stream:

    moe_route -> [moe_quantize_mx of x] -> moe_permute (maps only)
      -> moe_grouped_fc1_swiglu_dense -> moe_grouped_fc2_dense
         (routed experts, rows gathered through src_row, and the shared
         expert in the same launches)
      -> moe_combine

Without a shared expert, or when it cannot share the routed launches (fp32
layers, F_shared != F), the routed experts run through
moe_grouped_fc1_swiglu / moe_grouped_fc2 and the shared expert through the
same two calls with E = 1. The NVFP4 layer quantizes x with
moe_quantize_nvfp4 (operand values, fixed tensor scale) and runs
moe_grouped_fc1_swiglu_nvfp4 -> moe_grouped_fc2_nvfp4 (no shared expert).

MoEBackward runs the backward of the routed expert path (MXFP8), reusing
the forward's routing and maps, as one moe_grouped_mlp_bwd call, whose
steps are (and can also be issued one by one):

    moe_combine_bwd (dY rows, MX) -> moe_grouped_fc2_dgrad_dswiglu
      -> moe_grouped_fc1_dgrad -> moe_unpermute
      -> moe_quantize_mx_segments (dY, h, dA, x) -> moe_grouped_wgrad (dW2, dW1)

Intermediates that feed an MX quantization stay in fp32 (the saved fc1
output, dA, the dY products), so rounding happens only where the MX
operands are formed.

Only marshalling happens here; every step of the layer runs in the HIP
library.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib as L

FMT = {"fp32": L.MOE_F32, "bf16": L.MOE_BF16, "mxfp8": L.MOE_MXFP8_E4M3, "mxfp4": L.MOE_MXFP4_E2M1,
       "nvfp4": L.MOE_NVFP4_E2M1}


def is_mx(fmt: str) -> bool:
    return fmt in ("mxfp8", "mxfp4")


def code_cols(K: int, fmt: str) -> int:
    """Bytes per row of MX codes for K elements."""
    return K // 2 if fmt == "mxfp4" else K


def quantize_mx(t: torch.Tensor, fmt: str, stream=None):
    """MX-quantize a [..., K] fp32/bf16 tensor along its last axis with
    moe_quantize_mx. Returns (codes uint8 [..., K or K/2], scales uint8
    [..., K/32])."""
    K = t.shape[-1]
    rows = t.numel() // K
    codes = torch.empty(t.shape[:-1] + (code_cols(K, fmt),), dtype=torch.uint8, device=t.device)
    scales = torch.empty(t.shape[:-1] + (K // 32,), dtype=torch.uint8, device=t.device)
    L.moe_quantize_mx(t, L.fmt_of_dtype(t), rows, K, 0, FMT[fmt], codes, scales, stream)
    return codes, scales


def quantize_mx_t(t: torch.Tensor, fmt: str, stream=None):
    """MX-quantize each [R, K] bf16 matrix of a [..., R, K] tensor along R
    (moe_quantize_mx with axis 1), giving the transposed K-major copy:
    codes [..., K, R or R/2], scales [..., K, R/32]."""
    R, K = t.shape[-2], t.shape[-1]
    lead = t.shape[:-2]
    codes = torch.empty(lead + (K, code_cols(R, fmt)), dtype=torch.uint8, device=t.device)
    scales = torch.empty(lead + (K, R // 32), dtype=torch.uint8, device=t.device)
    flat_t, flat_c, flat_s = t.reshape(-1, R, K), codes.view(-1, K, codes.shape[-1]), \
        scales.view(-1, K, R // 32)
    for i in range(flat_t.shape[0]):
        L.moe_quantize_mx(flat_t[i], L.MOE_BF16, R, K, 1, FMT[fmt], flat_c[i], flat_s[i], stream)
    return codes, scales


def quantize_nvfp4(t: torch.Tensor, g: torch.Tensor, rows_per_tensor: int, codes=True,
                   vals=False, stream=None):
    """NVFP4-quantize a [..., K] fp32/bf16 tensor along its last axis with
    moe_quantize_nvfp4; row r uses tensor scale g[r // rows_per_tensor].
    Returns (codes uint8 [..., K/2] or None, scales uint8 [..., K/16] or
    None, vals bf16 [..., K] or None)."""
    K = t.shape[-1]
    rows = t.numel() // K
    lead = t.shape[:-1]
    c = torch.empty(lead + (K // 2,), dtype=torch.uint8, device=t.device) if codes else None
    sc = torch.empty(lead + (K // 16,), dtype=torch.uint8, device=t.device) if codes else None
    v = torch.empty(lead + (K,), dtype=torch.bfloat16, device=t.device) if vals else None
    L.moe_quantize_nvfp4(t, L.fmt_of_dtype(t), rows, K, rows_per_tensor, g, c, sc, v, stream)
    return c, sc, v


def nvfp4_tensor_scales(w: torch.Tensor, stream=None) -> torch.Tensor:
    """fp32 [E] tensor scales (amax / 2688) of the E matrices of w [E, N, K]
    (moe_nvfp4_tensor_scale)."""
    E = w.shape[0]
    g = torch.empty((E,), dtype=torch.float32, device=w.device)
    L.moe_nvfp4_tensor_scale(w, L.fmt_of_dtype(w), E, w[0].numel(), g, stream)
    return g


def pack_weights(codes: torch.Tensor, scales, fmt: str, half: int = 0, stream=None):
    """moe_pack_weights of [E, N, K] stored weights (bf16 values or MX codes
    with [E, N, K/32] scales) into the grouped GEMMs' streaming order.
    Returns (packed uint8 [E, bytes per expert], packed scales or None)."""
    E, N = codes.shape[0], codes.shape[1]
    K = codes.shape[2] * (2 if fmt in ("mxfp4", "nvfp4") else 1)
    nbytes = codes[0].numel() * codes.element_size()
    out = torch.empty((E, nbytes), dtype=torch.uint8, device=codes.device)
    out_sc = torch.empty_like(scales) if scales is not None else None
    L.moe_pack_weights(codes, scales, FMT[fmt], E, N, K, half, out, out_sc, stream)
    return out, out_sc


@dataclass
class ExpertWeights:
    """Expert weights as the grouped GEMMs consume them. fp32: plain w1
    [E, 2F, H] and w2 [E, H, F]. bf16 / MX: stored values (MX: E4M3 / E2M1
    codes with one E8M0 scale per 32 values along K) packed by
    moe_pack_weights, w1 with its gate/up halves paired. With
    `transposed`, also the copies the backward's data-gradient GEMMs
    contract over: w1t [E, H, 2F] (blocks along 2F) and w2t [E, F, H]
    (blocks along H), quantized from the same masters and packed. NVFP4:
    E2M1 codes with E4M3 scales per 16 values along K, packed, and each
    expert matrix's fp32 tensor scale in w1_g / w2_g [E]."""
    w1: torch.Tensor
    w2: torch.Tensor
    w1_sc: torch.Tensor | None = None
    w2_sc: torch.Tensor | None = None
    w1t: torch.Tensor | None = None
    w2t: torch.Tensor | None = None
    w1t_sc: torch.Tensor | None = None
    w2t_sc: torch.Tensor | None = None
    w1_g: torch.Tensor | None = None
    w2_g: torch.Tensor | None = None

    @staticmethod
    def from_dense(w1: torch.Tensor, w2: torch.Tensor, fmt: str, stream=None,
                   transposed: bool = False) -> "ExpertWeights":
        if fmt == "fp32":
            if transposed:
                raise ValueError("transposed weight copies are built for MX formats only")
            return ExpertWeights(w1, w2)
        if w1.dim() == 2:                     # a single (shared) expert
            w1, w2 = w1.unsqueeze(0), w2.unsqueeze(0)
        F = w1.shape[1] // 2
        if fmt == "bf16":
            if transposed:
                raise ValueError("transposed weight copies are built for MX formats only")
            p1, _ = pack_weights(w1, None, fmt, F, stream)
            p2, _ = pack_weights(w2, None, fmt, 0, stream)
            return ExpertWeights(p1, p2)
        if fmt == "nvfp4":
            if transposed:
                raise ValueError("the NVFP4 layer runs the forward only")
            gs, packed = [], []
            for w, half in ((w1, F), (w2, 0)):
                g = nvfp4_tensor_scales(w, stream)
                c, sc, _ = quantize_nvfp4(w, g, w.shape[1], stream=stream)
                packed.append(pack_weights(c, sc, fmt, half, stream))
                gs.append(g)
                del c, sc
            (p1, q1), (p2, q2) = packed
            return ExpertWeights(p1, p2, q1, q2, w1_g=gs[0], w2_g=gs[1])
        c1, s1 = quantize_mx(w1, fmt, stream)
        c2, s2 = quantize_mx(w2, fmt, stream)
        p1, q1 = pack_weights(c1, s1, fmt, F, stream)
        p2, q2 = pack_weights(c2, s2, fmt, 0, stream)
        del c1, s1, c2, s2
        ew = ExpertWeights(p1, p2, q1, q2)
        if transposed:
            c, sc = quantize_mx_t(w1, fmt, stream)
            ew.w1t, ew.w1t_sc = pack_weights(c, sc, fmt, 0, stream)
            del c, sc
            c, sc = quantize_mx_t(w2, fmt, stream)
            ew.w2t, ew.w2t_sc = pack_weights(c, sc, fmt, 0, stream)
        return ew

    @property
    def E(self) -> int:
        return self.w1.shape[0]


class MoEForward:
    def __init__(self, *, T, H, F, E, n_group, topk_group, k, routed_scale, fmt,
                 F_shared=0, align=1, device="cuda", keep_logits=False, save_act=False,
                 fuse_shared=None, x_global=0.0, h_global=0.0):
        """fuse_shared: run the shared expert inside the routed fc1 / fc2
        launches (its tiles fill the matrix cores while the routed tiles
        stream weights). Default: whenever the shared expert has the routed
        experts' width and the layer is not fp32. x_global / h_global: the
        NVFP4 layer's fixed tensor scales of the hidden states and of h."""
        self.T, self.H, self.F, self.E = T, H, F, E
        self.n_group, self.topk_group, self.k = n_group, topk_group, k
        self.routed_scale, self.fmt, self.F_shared, self.align = routed_scale, fmt, F_shared, align
        dev = torch.device(device)
        act = torch.float32 if fmt == "fp32" else torch.bfloat16
        self.act_dtype = act
        self.act_fmt = FMT["fp32"] if fmt == "fp32" else FMT["bf16"]
        i32 = dict(dtype=torch.int32, device=dev)
        self.logits = torch.empty((T, E), dtype=torch.float32, device=dev) if keep_logits else None
        self.route_ws = torch.empty((max(1, L.moe_route_workspace(T, H, E)),), dtype=torch.uint8,
                                    device=dev)
        self.topk_idx = torch.empty((T, k), **i32)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.counts = torch.empty((E,), **i32)
        self.offsets = torch.empty((E + 1,), **i32)
        self.row_map = torch.empty((T, k), **i32)
        self.bound = L.moe_permute_rows_bound(T, k, E, align)
        self.src_row = torch.empty((max(1, self.bound),), **i32)
        self.perm_ws = torch.empty((max(1, L.moe_permute_workspace(T, k, E)),), dtype=torch.uint8, device=dev)
        if is_mx(fmt):
            self.xq = torch.empty((T, code_cols(H, fmt)), dtype=torch.uint8, device=dev)
            self.xq_sc = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
        elif fmt == "nvfp4":
            if not (x_global > 0 and h_global > 0):
                raise ValueError("the NVFP4 layer needs positive x_global and h_global")
            if F_shared:
                raise ValueError("the NVFP4 layer has no shared expert")
            # operand values of x (code * scale) and its tensor scale
            self.xq = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
            self.xq_sc = None
            self.x_g = torch.full((1,), x_global, dtype=torch.float32, device=dev)
        else:
            self.xq = self.xq_sc = None
        self.x_global, self.h_global = x_global, h_global
        can_fuse = bool(F_shared) and F_shared == F and fmt not in ("fp32", "nvfp4") and T > 0
        if fuse_shared is None:
            fuse_shared = can_fuse
        if fuse_shared and not can_fuse:
            raise ValueError("the shared expert folds into the routed launches only when "
                             "F_shared == F, T > 0 and the layer is not fp32")
        self.fuse_shared = fuse_shared
        # with the shared expert folded in, its rows follow the routed rows
        rows = max(1, self.bound) + (T if fuse_shared else 0)
        self.y_rows = torch.empty((rows, H), dtype=act, device=dev)
        self.h, self.h_sc = self._h_buffers(rows, F, dev)
        # fc1 output (gate | up) per expert row in fp32, kept for the backward
        self.act_save = (torch.empty((max(1, self.bound), 2 * F), dtype=torch.float32, device=dev)
                         if save_act else None)
        if fuse_shared:
            self.y_shared = self.y_rows[self.bound:self.bound + T]
        elif F_shared:
            self.shared_offsets = torch.tensor([0, T], **i32)
            self.y_shared = torch.empty((T, H), dtype=act, device=dev)
            self.hs, self.hs_sc = self._h_buffers(max(1, T), F_shared, dev)
        else:
            self.y_shared = None
        self.out = torch.empty((T, H), dtype=act, device=dev)

    def _h_buffers(self, rows, F, dev):
        """SwiGLU output rows in the layer format (+ MX scales)."""
        if is_mx(self.fmt):
            return (torch.empty((rows, code_cols(F, self.fmt)), dtype=torch.uint8, device=dev),
                    torch.empty((rows, F // 32), dtype=torch.uint8, device=dev))
        # bf16 values (NVFP4: operand values code * scale)
        return torch.empty((rows, F), dtype=self.act_dtype, device=dev), None

    def route(self, x, w_router, bias, logits_in=None, stream=None):
        L.moe_route(x, self.act_fmt, w_router, bias, logits_in, self.T, self.H, self.E, self.n_group,
                    self.topk_group, self.k, self.routed_scale, self.logits, self.topk_idx,
                    self.topk_w, None if logits_in is not None else self.route_ws, stream)

    def quantize_x(self, x, stream=None):
        if is_mx(self.fmt):
            L.moe_quantize_mx(x, self.act_fmt, self.T, self.H, 0, FMT[self.fmt], self.xq, self.xq_sc,
                              stream)
        elif self.fmt == "nvfp4" and self.T > 0:
            L.moe_quantize_nvfp4(x, self.act_fmt, self.T, self.H, self.T, self.x_g, None, None,
                                 self.xq, stream)

    def permute(self, stream=None):
        L.moe_permute(self.topk_idx, self.T, self.k, self.E, self.align, None, 0, None, 0,
                      self.counts, self.offsets, self.row_map, self.src_row, None, None,
                      self.perm_ws, stream)

    def experts_fc1(self, x, ew: ExpertWeights, stream=None, sw: ExpertWeights | None = None):
        """Routed fc1 + SwiGLU; with fuse_shared also the shared expert's
        (sw required)."""
        if self.fmt == "nvfp4":
            if self.act_save is not None:
                raise ValueError("the NVFP4 layer keeps no fc1 output")
            L.moe_grouped_fc1_swiglu_nvfp4(self.xq, self.src_row, ew.w1, ew.w1_sc, ew.w1_g,
                                           self.x_global, self.h_global, self.offsets, self.E,
                                           self.H, self.F, self.bound, self.h, stream)
            return
        a, a_sc = (self.xq, self.xq_sc) if is_mx(self.fmt) else (x, None)
        f = FMT[self.fmt]
        if self.fuse_shared:
            L.moe_grouped_fc1_swiglu_dense(a, a_sc, f, self.src_row, ew.w1, ew.w1_sc, f,
                                           self.offsets, self.E, self.H, self.F, self.bound,
                                           self.act_save, self.h, self.h_sc, sw.w1, sw.w1_sc,
                                           self.T, stream)
        else:
            L.moe_grouped_fc1_swiglu(a, a_sc, f, self.src_row, ew.w1, ew.w1_sc, f, self.offsets,
                                     self.E, self.H, self.F, self.bound, self.act_save, self.h,
                                     self.h_sc, stream)

    def experts_fc2(self, ew: ExpertWeights, stream=None, sw: ExpertWeights | None = None):
        if self.fmt == "nvfp4":
            L.moe_grouped_fc2_nvfp4(self.h, ew.w2, ew.w2_sc, ew.w2_g, self.h_global, self.offsets,
                                    self.E, self.H, self.F, self.bound, self.y_rows, stream)
            return
        f = FMT[self.fmt]
        if self.fuse_shared:
            L.moe_grouped_fc2_dense(self.h, self.h_sc, f, ew.w2, ew.w2_sc, f, self.offsets,
                                    self.E, self.H, self.F, self.bound, self.y_rows, self.act_fmt,
                                    sw.w2, sw.w2_sc, self.T, stream)
        else:
            L.moe_grouped_fc2(self.h, self.h_sc, f, ew.w2, ew.w2_sc, f, self.offsets, self.E,
                              self.H, self.F, self.bound, self.y_rows, self.act_fmt, stream)

    def experts(self, x, ew: ExpertWeights, stream=None, sw: ExpertWeights | None = None):
        self.experts_fc1(x, ew, stream, sw)
        self.experts_fc2(ew, stream, sw)

    def shared(self, x, sw: ExpertWeights, stream=None):
        """The shared expert on its own (only when it is not folded into the
        routed launches)."""
        if self.fuse_shared:
            raise RuntimeError("the shared expert runs inside experts_fc1 / experts_fc2")
        a, a_sc = (self.xq, self.xq_sc) if is_mx(self.fmt) else (x, None)
        f = FMT[self.fmt]
        L.moe_grouped_fc1_swiglu(a, a_sc, f, None, sw.w1, sw.w1_sc, f, self.shared_offsets, 1,
                                 self.H, self.F_shared, self.T, None, self.hs, self.hs_sc, stream)
        L.moe_grouped_fc2(self.hs, self.hs_sc, f, sw.w2, sw.w2_sc, f, self.shared_offsets, 1,
                          self.H, self.F_shared, self.T, self.y_shared, self.act_fmt, stream)

    def combine(self, stream=None):
        L.moe_combine(self.y_rows, self.act_fmt, self.row_map, self.topk_w, self.y_shared, self.T,
                      self.k, self.H, self.out, self.act_fmt, stream)

    def __call__(self, x, w_router, bias, ew: ExpertWeights, sw: ExpertWeights | None = None,
                 stream=None):
        """The whole forward; returns the preallocated output [T, H]."""
        self.route(x, w_router, bias, stream=stream)
        self.quantize_x(x, stream)
        self.permute(stream)
        self.experts(x, ew, stream, sw)
        if self.F_shared and not self.fuse_shared:
            self.shared(x, sw, stream)
        self.combine(stream)
        return self.out

    @classmethod
    def for_config(cls, cfg, device="cuda", keep_logits=False, T=None, save_act=False,
                   fuse_shared=None):
        return cls(T=cfg.T if T is None else T, H=cfg.H, F=cfg.F, E=cfg.E, n_group=cfg.n_group,
                   topk_group=cfg.topk_group, k=cfg.k, routed_scale=cfg.routed_scale, fmt=cfg.fmt,
                   F_shared=cfg.F_shared if cfg.n_shared else 0, align=cfg.align, device=device,
                   keep_logits=keep_logits, save_act=save_act, fuse_shared=fuse_shared,
                   x_global=cfg.x_global, h_global=cfg.h_global)


class MoEBackward:
    """Backward of the routed experts of one MoEForward pass (built with
    save_act=True, MXFP8). Produces dx [T, H] (gradient through the routed
    experts) and the weight gradients dw1 [E, 2F, H], dw2 [E, H, F] (bf16).
    Routing weights are constants and the quantizers pass gradients straight
    through.

    Calling the object runs the whole backward as one moe_grouped_mlp_bwd
    call on a preallocated workspace. The step methods (data_grad,
    operands_dw2, gemm_dw2, operands_dw1, gemm_dw1) issue the same kernels
    one C call at a time on buffers of their own (allocated on first use),
    so each step can be timed or checked by itself."""

    def __init__(self, fwd: MoEForward):
        if fwd.fmt != "mxfp8":
            raise ValueError("the backward runs in MXFP8")
        if fwd.act_save is None:
            raise ValueError("the forward must keep its fc1 output (save_act=True)")
        self.fwd = fwd
        T, H, F, E, bound = fwd.T, fwd.H, fwd.F, fwd.E, max(1, fwd.bound)
        dev = fwd.topk_idx.device
        self.dev = dev
        bf = dict(dtype=fwd.act_dtype, device=dev)
        self.dx = torch.empty((T, H), **bf)
        self.dw1 = torch.empty((E, 2 * F, H), dtype=torch.bfloat16, device=dev)
        self.dw2 = torch.empty((E, H, F), dtype=torch.bfloat16, device=dev)
        nws = L.moe_grouped_mlp_bwd_workspace(T, fwd.k, E, H, F, bound, FMT["mxfp8"])
        if nws == 0:
            raise ValueError("moe_grouped_mlp_bwd does not support these sizes")
        self.ws = torch.empty((nws,), dtype=torch.uint8, device=dev)
        self._staged = False

    def stage_buffers(self):
        """Buffers of the one-call-per-step path."""
        if self._staged:
            return
        fwd, dev = self.fwd, self.dev
        H, F, E, bound = fwd.H, fwd.F, fwd.E, max(1, fwd.bound)
        u8 = dict(dtype=torch.uint8, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        self.dy_q = torch.empty((bound, H), **u8)
        self.dy_sc = torch.empty((bound, H // 32), **u8)
        self.row_w = torch.empty((bound,), **f32)
        self.da = torch.empty((bound, 2 * F), **u8)
        self.da_sc = torch.empty((bound, 2 * F // 32), **u8)
        self.da_f32 = torch.empty((bound, 2 * F), **f32)
        self.dx_perm = torch.empty((bound, H), dtype=torch.bfloat16, device=dev)
        ks = L.moe_segments_kstride(fwd.bound, E)
        self.kstride = ks
        self.kofs = torch.empty((E + 1,), dtype=torch.int32, device=dev)
        self.dyT, self.dyT_sc = torch.empty((H, ks), **u8), torch.empty((H, ks // 32), **u8)
        self.hT, self.hT_sc = torch.empty((F, ks), **u8), torch.empty((F, ks // 32), **u8)
        self.daT, self.daT_sc = torch.empty((2 * F, ks), **u8), torch.empty((2 * F, ks // 32), **u8)
        self.xT, self.xT_sc = torch.empty((H, ks), **u8), torch.empty((H, ks // 32), **u8)
        self._staged = True

    def data_grad(self, dout, ew: ExpertWeights, stream=None):
        """dY rows -> dA (SwiGLU backward fused) -> dX rows -> dx."""
        self.stage_buffers()
        f, fw = FMT["mxfp8"], self.fwd
        T, H, F, E, k, rows = fw.T, fw.H, fw.F, fw.E, fw.k, fw.bound
        L.moe_combine_bwd(dout, fw.act_fmt, fw.row_map, fw.src_row, fw.topk_w, T, k, H, rows,
                          self.dy_q, f, self.dy_sc, self.row_w, stream)
        L.moe_grouped_fc2_dgrad_dswiglu(self.dy_q, self.dy_sc, f, ew.w2t, ew.w2t_sc, fw.offsets,
                                        E, H, F, rows, fw.act_save, self.da, self.da_sc,
                                        self.da_f32, stream)
        L.moe_grouped_fc1_dgrad(self.da, self.da_sc, f, ew.w1t, ew.w1t_sc, fw.offsets, E, H, F,
                                rows, self.dx_perm, stream)
        L.moe_unpermute(self.dx_perm, L.MOE_BF16, fw.row_map, T, k, H, self.dx, fw.act_fmt, stream)

    def _seg(self, src, in_fmt, mode, scale, C, codes, scales, stream):
        fw = self.fwd
        L.moe_quantize_mx_segments(src, in_fmt, mode, fw.src_row, fw.offsets, scale, fw.E,
                                   fw.bound, C, self.kstride, FMT["mxfp8"], codes, scales,
                                   self.kofs, stream)

    def operands_dw2(self, dout, stream=None):
        """The dW2 operands in the stage-major segment layout: dY rows formed
        as w * dout, h recomputed from the saved fc1 output, both MX
        quantized along the rows of each expert segment."""
        self.stage_buffers()
        fw = self.fwd
        self._seg(dout, fw.act_fmt, 1, self.row_w, fw.H, self.dyT, self.dyT_sc, stream)
        self._seg(fw.act_save, L.MOE_F32, 2, None, fw.F, self.hT, self.hT_sc, stream)

    def gemm_dw2(self, stream=None):
        """dW2 = dY^T h per expert, contracting over the expert's rows."""
        fw = self.fwd
        L.moe_grouped_wgrad(self.dyT, self.dyT_sc, self.hT, self.hT_sc, FMT["mxfp8"], self.kofs,
                            fw.E, fw.H, fw.F, self.kstride, self.dw2, stream)

    def operands_dw1(self, x, stream=None):
        """The dW1 operands: dA (its fp32 copy) and the token rows x."""
        self.stage_buffers()
        fw = self.fwd
        self._seg(self.da_f32, L.MOE_F32, 0, None, 2 * fw.F, self.daT, self.daT_sc, stream)
        self._seg(x, fw.act_fmt, 1, None, fw.H, self.xT, self.xT_sc, stream)

    def gemm_dw1(self, stream=None):
        """dW1 = dA^T x per expert, contracting over the expert's rows."""
        fw = self.fwd
        L.moe_grouped_wgrad(self.daT, self.daT_sc, self.xT, self.xT_sc, FMT["mxfp8"], self.kofs,
                            fw.E, 2 * fw.F, fw.H, self.kstride, self.dw1, stream)

    def staged(self, dout, x, ew: ExpertWeights, stream=None):
        """The whole backward one C call per step."""
        self.data_grad(dout, ew, stream)
        self.operands_dw2(dout, stream)
        self.gemm_dw2(stream)
        self.operands_dw1(x, stream)
        self.gemm_dw1(stream)
        return self.dx, self.dw1, self.dw2

    def __call__(self, dout, x, ew: ExpertWeights, stream=None):
        """The whole backward in one moe_grouped_mlp_bwd call."""
        fw = self.fwd
        L.moe_grouped_mlp_bwd(dout, x, fw.act_fmt, fw.row_map, fw.src_row, fw.topk_w, fw.offsets,
                              fw.act_save, ew.w1t, ew.w1t_sc, ew.w2t, ew.w2t_sc, FMT["mxfp8"], fw.T,
                              fw.k, fw.E, fw.H, fw.F, max(1, fw.bound), self.dx, self.dw1,
                              self.dw2, self.ws, stream)
        return self.dx, self.dw1, self.dw2


class RouterBackward:
    """Router backward of one MoEForward pass (bf16 layer built with
    keep_logits=True): the combine-weight gradient against the forward's
    expert output rows, pulled back through the weight normalization and the
    sigmoid into the logits (plus, with aux_alpha, the sequence-wise balance
    loss over sequences of seq_len tokens), then into the hidden states
    (dx [T, H] bf16) and the router weight (dw [E, H] fp32), in one
    moe_route_bwd call."""

    def __init__(self, fwd: MoEForward, seq_len: int = 0, aux_alpha: float = 0.0):
        if fwd.logits is None:
            raise ValueError("the forward must keep its router logits (keep_logits=True)")
        if fwd.act_fmt != L.MOE_BF16:
            raise ValueError("the router backward runs on bf16 layers")
        self.fwd, self.seq_len, self.aux_alpha = fwd, seq_len, aux_alpha
        T, H, E = fwd.T, fwd.H, fwd.E
        dev = fwd.topk_idx.device
        nws = L.moe_route_bwd_workspace(max(1, T), H, E, seq_len if aux_alpha else 0)
        if nws == 0:
            raise ValueError("moe_route_bwd does not support these sizes")
        self.ws = torch.empty((nws,), dtype=torch.uint8, device=dev)
        self.dlogits = torch.empty((T, E), dtype=torch.float32, device=dev)
        self.aux_loss = torch.zeros((1,), dtype=torch.float32, device=dev)
        self.dx = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        self.dw = torch.empty((E, H), dtype=torch.float32, device=dev)

    def __call__(self, dout, x, w_router, stream=None):
        fw = self.fwd
        L.moe_route_bwd(dout, fw.y_rows, fw.act_fmt, fw.row_map, fw.topk_idx, fw.logits, x,
                        w_router, fw.T, fw.k, fw.E, fw.H, fw.routed_scale, self.seq_len,
                        self.aux_alpha, self.dlogits, self.aux_loss if self.aux_alpha else None,
                        self.dx, self.dw, self.ws, stream)
        return self.dx, self.dw


def bias_update(fwd: MoEForward, bias: torch.Tensor, gamma: float, out=None, stream=None):
    """The aux-loss-free bias update from the pass's expert loads
    (moe_bias_update); in place unless `out` is given."""
    out = bias if out is None else out
    L.moe_bias_update(fwd.counts, fwd.E, gamma, bias, out, stream)
    return out
