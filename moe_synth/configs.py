"""Workload definitions for the sigmoid-routed MoE layer.

Pure data: shapes, routing hyper-parameters and the statistics of the
synthetic inputs. No arithmetic of the method lives here.

Page abbreviations used in citations:
  [TE-DSV3]  "[PyTorch] DeepSeekV3Layer: full MoE transformer layer
             (MLA + DeepSeek MoE)" (TransformerEngine pull request page)
  [AIC-DSV4] "[Support Matrix] DeepSeek-V4 support on trtllm ..."
             (aiconfigurator issue page)
  [SGL-NVFP4] "Mistral Large 3 NVFP4 TRTLLM MoE support" (sglang pull
             request page)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class MoEConfig:
    name: str
    family: str          # inputs of configs in one family share seeds
    T: int               # tokens
    H: int               # hidden size (fc1 contraction, fc2 output)
    F: int               # expert FFN size (fc1 -> 2F, fc2 contraction)
    E: int               # routed experts
    n_group: int
    topk_group: int
    k: int
    routed_scale: float
    n_shared: int        # 0 or 1 shared expert
    F_shared: int
    fmt: str             # 'fp32' | 'bf16' | 'mxfp8' | 'mxfp4' | 'nvfp4'
    x_std: float
    router_std: float
    bias_kind: str       # 'uniform' | 'zipf'
    bias_range: float    # half-width of U(-r, r) for 'uniform'
    backward: bool = False
    align: int = 1       # padding granule of each expert segment
    zipf_s: float = 1.1
    n_zero_experts: int = 0
    x_rows_from: str = ""  # reuse the first T rows of another config's x
    # NVFP4 layer: fixed tensor scales of the hidden states and of h
    x_global: float = 0.0
    h_global: float = 0.0

    @property
    def rows(self) -> int:
        return self.T * self.k

    @property
    def act_dtype(self) -> str:
        """Storage type of hidden states and outputs."""
        return "fp32" if self.fmt == "fp32" else "bf16"

    @property
    def w1_std(self) -> float:
        return 1.0 / math.sqrt(self.H)

    @property
    def w2_std(self) -> float:
        return 1.0 / math.sqrt(self.F)

    @property
    def w2s_std(self) -> float:
        return 1.0 / math.sqrt(self.F_shared)

    def flops_forward(self) -> float:
        """2*M*N*K over router GEMM, routed fc1+fc2 on unpadded rows and the
        shared expert; elementwise work is not counted."""
        f = 2.0 * self.T * self.H * self.E
        f += 2.0 * self.rows * self.H * (2 * self.F) + 2.0 * self.rows * self.F * self.H
        if self.n_shared:
            f += 2.0 * self.T * self.H * (2 * self.F_shared) + 2.0 * self.T * self.F_shared * self.H
        return f

    def flops_backward(self) -> float:
        """fc2-dgrad, fc1-dgrad, dW2 and dW1 over the unpadded rows."""
        R = self.rows
        return 2.0 * R * self.H * self.F + 2.0 * R * 2 * self.F * self.H \
            + 2.0 * R * self.H * self.F + 2.0 * R * 2 * self.F * self.H


# -- the five workloads ------------------------------------------------------
# Tiny fp32 layer: 16 experts in 4 groups, top-4 from the top-2 groups.
TINY_FP32 = MoEConfig(
    name="tiny_fp32", family="tiny", T=64, H=256, F=128, E=16, n_group=4,
    topk_group=2, k=4, routed_scale=1.0, n_shared=0, F_shared=0, fmt="fp32",
    x_std=1.0 / math.sqrt(256), router_std=1.0 / math.sqrt(256),
    bias_kind="uniform", bias_range=0.1)
# Same layer with unit-variance hidden states, so every expert is used.
TINY_FP32_UNITX = replace(TINY_FP32, name="tiny_fp32_unitx", x_std=1.0)

# DeepSeek-V3 dims (the [TE-DSV3] Performance section measures these dims),
# bf16, 4096 tokens, grouped top-8, routed scale 2.5, one shared expert.
DSV3_BF16 = MoEConfig(
    name="dsv3_bf16_t4096", family="dsv3", T=4096, H=7168, F=2048, E=256,
    n_group=8, topk_group=4, k=8, routed_scale=2.5, n_shared=1, F_shared=2048,
    fmt="bf16", x_std=1.0, router_std=1.0 / math.sqrt(7168),
    bias_kind="uniform", bias_range=0.05)
# Decode shape of the same layer: 64 tokens, MXFP8 weights and activations.
DSV3_MXFP8_DECODE = replace(
    DSV3_BF16, name="dsv3_mxfp8_decode_t64", T=64, fmt="mxfp8",
    x_rows_from="dsv3_bf16_t4096")
# DeepSeek-V4 expert geometry 4096/2048/top-6/e256 ([AIC-DSV4] per-op status
# table, moe row), MXFP4 W4A4 (the 4-bit W4A4 path of [SGL-NVFP4]).
DSV4_MXFP4 = MoEConfig(
    name="dsv4_mxfp4_t16384", family="dsv4a", T=16384, H=4096, F=2048, E=256,
    n_group=1, topk_group=1, k=6, routed_scale=1.0, n_shared=0, F_shared=0,
    fmt="mxfp4", x_std=1.0, router_std=1.0 / math.sqrt(4096),
    bias_kind="uniform", bias_range=0.05)
# DeepSeek-V4 expert geometry 7168/3072/top-6/e384, MXFP8, Zipf-skewed
# expert popularity, forward and backward.
DSV4_SKEW_MXFP8 = MoEConfig(
    name="dsv4_skew_mxfp8_t8192", family="dsv4b", T=8192, H=7168, F=3072,
    E=384, n_group=1, topk_group=1, k=6, routed_scale=1.0, n_shared=0,
    F_shared=0, fmt="mxfp8", x_std=1.0, router_std=1.0 / math.sqrt(7168),
    bias_kind="zipf", bias_range=0.0, backward=True, align=32, zipf_s=1.1,
    n_zero_experts=8)

# One expert-parallel rank's share at DeepSeek-V3 dims ([TE-DSV3] Performance
# section, setup: 8 experts per rank, top-k 8, 4096 tokens per rank): the 8
# local experts each receive 4096 rows, here from 4096 tokens routed top-8
# over exactly those 8 experts, MXFP8 forward and backward (the fused
# grouped MLP's fc1+SwiGLU, fc2, dGLU and wgrad). No shared expert: the
# pages time it with the dense GEMMs, not the grouped MLP.
DSV3_EP_SHARE = MoEConfig(
    name="dsv3_ep8_mxfp8_t4096", family="dsv3_ep8", T=4096, H=7168, F=2048,
    E=8, n_group=1, topk_group=1, k=8, routed_scale=2.5, n_shared=0,
    F_shared=0, fmt="mxfp8", x_std=1.0, router_std=1.0 / math.sqrt(7168),
    bias_kind="uniform", bias_range=0.05, backward=True, align=32)

# The same layer with NVFP4 W4A4 ([SGL-NVFP4] title and Modifications: the
# 4-bit format the pages run): E2M1 values, E4M3 scales per 16, one fp32
# scale per tensor; the activation scales are fixed for the workload (2^-8
# for N(0,1) hidden states: nothing saturates below 6 * 448 * 2^-8 = 10.5;
# 2^-6 for h).
DSV4_NVFP4 = replace(DSV4_MXFP4, name="dsv4_nvfp4_t16384", fmt="nvfp4",
                     x_global=2.0 ** -8, h_global=2.0 ** -6)

# -- reduced shapes of the same structure, small enough for full parity ----
# (several GEMM tiles along every axis, ragged token counts)
MINI_BF16 = replace(
    DSV3_BF16, name="mini_bf16", family="mini_bf16", T=300, H=512, F=256,
    E=32, F_shared=256, router_std=1.0 / math.sqrt(512))
MINI_MXFP8_DECODE = replace(
    MINI_BF16, name="mini_mxfp8_decode", family="mini_bf16", T=40,
    fmt="mxfp8", x_rows_from="mini_bf16")
MINI_MXFP4 = replace(
    DSV4_MXFP4, name="mini_mxfp4", family="mini_mxfp4", T=500, H=512, F=256,
    E=32, router_std=1.0 / math.sqrt(512))
MINI_SKEW = replace(
    DSV4_SKEW_MXFP8, name="mini_skew_mxfp8", family="mini_skew", T=300,
    H=512, F=384, E=48, router_std=1.0 / math.sqrt(512), n_zero_experts=2)
MINI_EP_SHARE = replace(
    DSV3_EP_SHARE, name="mini_ep8_mxfp8", family="mini_ep8", T=300, H=512, F=256,
    router_std=1.0 / math.sqrt(512))
MINI_NVFP4 = replace(
    DSV4_NVFP4, name="mini_nvfp4", family="mini_mxfp4", T=500, H=512, F=256,
    E=32, router_std=1.0 / math.sqrt(512))
MINI_FP32 = replace(
    TINY_FP32, name="mini_fp32", family="mini_fp32", T=333, H=320, F=192,
    E=24, n_group=6, topk_group=3, k=5, x_std=1.0,
    router_std=1.0 / math.sqrt(320))

ALL = {c.name: c for c in (
    TINY_FP32, TINY_FP32_UNITX, DSV3_BF16, DSV3_MXFP8_DECODE, DSV4_MXFP4,
    DSV4_SKEW_MXFP8, DSV3_EP_SHARE, DSV4_NVFP4, MINI_BF16, MINI_MXFP8_DECODE,
    MINI_MXFP4, MINI_SKEW, MINI_EP_SHARE, MINI_NVFP4, MINI_FP32)}

# The workload the headline throughput is quoted on.
HEADLINE = DSV3_BF16


def get(name: str) -> MoEConfig:
    return ALL[name]
