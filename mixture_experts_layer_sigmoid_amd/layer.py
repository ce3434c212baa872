"""One forward pass of the routed MoE layer as a sequence of C-ABI calls.

The object preallocates every buffer the pass needs (torch device memory)
and then issues, on one stream:

    moe_route -> [moe_quantize_mx of x] -> moe_permute (maps only)
      -> moe_grouped_mlp_fwd (routed experts, rows gathered through src_row)
      -> [moe_grouped_mlp_fwd for the shared expert, E = 1]
      -> moe_combine

Only marshalling happens here; every step of the layer runs in the HIP
library.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib as L

FMT = {"fp32": L.MOE_F32, "bf16": L.MOE_BF16, "mxfp8": L.MOE_MXFP8_E4M3, "mxfp4": L.MOE_MXFP4_E2M1}


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


@dataclass
class ExpertWeights:
    """Stored expert weights: w1 [E, 2F, H], w2 [E, H, F] in the layer
    format (MX: codes, with scales w1_sc [E, 2F, H/32], w2_sc [E, H, F/32])."""
    w1: torch.Tensor
    w2: torch.Tensor
    w1_sc: torch.Tensor | None = None
    w2_sc: torch.Tensor | None = None

    @staticmethod
    def from_dense(w1: torch.Tensor, w2: torch.Tensor, fmt: str, stream=None) -> "ExpertWeights":
        if not is_mx(fmt):
            return ExpertWeights(w1, w2)
        c1, s1 = quantize_mx(w1, fmt, stream)
        c2, s2 = quantize_mx(w2, fmt, stream)
        return ExpertWeights(c1, c2, s1, s2)


class MoEForward:
    def __init__(self, *, T, H, F, E, n_group, topk_group, k, routed_scale, fmt,
                 F_shared=0, align=1, device="cuda", keep_logits=False):
        self.T, self.H, self.F, self.E = T, H, F, E
        self.n_group, self.topk_group, self.k = n_group, topk_group, k
        self.routed_scale, self.fmt, self.F_shared, self.align = routed_scale, fmt, F_shared, align
        dev = torch.device(device)
        act = torch.float32 if fmt == "fp32" else torch.bfloat16
        self.act_dtype = act
        self.act_fmt = FMT["fp32"] if fmt == "fp32" else FMT["bf16"]
        i32 = dict(dtype=torch.int32, device=dev)
        self.logits = torch.empty((T, E), dtype=torch.float32, device=dev) if keep_logits else None
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
        else:
            self.xq = self.xq_sc = None
        self.y_rows = torch.empty((max(1, self.bound), H), dtype=act, device=dev)
        self.h, self.h_sc = self._h_buffers(max(1, self.bound), F, dev)
        if F_shared:
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
        return torch.empty((rows, F), dtype=self.act_dtype, device=dev), None

    def route(self, x, w_router, bias, logits_in=None, stream=None):
        L.moe_route(x, self.act_fmt, w_router, bias, logits_in, self.T, self.H, self.E, self.n_group,
                    self.topk_group, self.k, self.routed_scale, self.logits, self.topk_idx,
                    self.topk_w, stream)

    def quantize_x(self, x, stream=None):
        if is_mx(self.fmt):
            L.moe_quantize_mx(x, self.act_fmt, self.T, self.H, 0, FMT[self.fmt], self.xq, self.xq_sc,
                              stream)

    def permute(self, stream=None):
        L.moe_permute(self.topk_idx, self.T, self.k, self.E, self.align, None, 0, None, 0,
                      self.counts, self.offsets, self.row_map, self.src_row, None, None,
                      self.perm_ws, stream)

    def experts_fc1(self, x, ew: ExpertWeights, stream=None):
        a, a_sc = (self.xq, self.xq_sc) if is_mx(self.fmt) else (x, None)
        f = FMT[self.fmt]
        L.moe_grouped_fc1_swiglu(a, a_sc, f, self.src_row, ew.w1, ew.w1_sc, f, self.offsets, self.E,
                                 self.H, self.F, self.bound, None, self.h, self.h_sc, stream)

    def experts_fc2(self, ew: ExpertWeights, stream=None):
        f = FMT[self.fmt]
        L.moe_grouped_fc2(self.h, self.h_sc, f, ew.w2, ew.w2_sc, f, self.offsets, self.E, self.H,
                          self.F, self.bound, self.y_rows, self.act_fmt, stream)

    def experts(self, x, ew: ExpertWeights, stream=None):
        self.experts_fc1(x, ew, stream)
        self.experts_fc2(ew, stream)

    def shared(self, x, sw: ExpertWeights, stream=None):
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
        self.experts(x, ew, stream)
        if self.F_shared:
            self.shared(x, sw, stream)
        self.combine(stream)
        return self.out

    @classmethod
    def for_config(cls, cfg, device="cuda", keep_logits=False, T=None):
        return cls(T=cfg.T if T is None else T, H=cfg.H, F=cfg.F, E=cfg.E, n_group=cfg.n_group,
                   topk_group=cfg.topk_group, k=cfg.k, routed_scale=cfg.routed_scale, fmt=cfg.fmt,
                   F_shared=cfg.F_shared if cfg.n_shared else 0, align=cfg.align, device=device,
                   keep_logits=keep_logits)
