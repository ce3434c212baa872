"""NVFP4 block quantization: E2M1 elements, one E4M3 scale per 16 values,
one fp32 scale per tensor.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this.

[SGL-NVFP4] (title, Modifications: a W4A4 NVFP4 MoE) names the format but
prints no layout or recipe; the readings taken are the public NVFP4
definition and its usual two-level recipe:
  * value = e2m1(code) * e4m3(block scale) * g, blocks of 16 consecutive
    values along the contraction axis, g one fp32 value per tensor (per
    expert weight matrix; for activations a fixed per-layer constant, as a
    deployment calibrates it);
  * a weight tensor's g = fp32(amax / 2688) (2688 = 6 * 448, the largest
    E2M1 value times the largest E4M3 value), 1 when amax == 0;
  * block scale: t = fp32(amax_block / fp32(6 g)), rounded to the nearest
    E4M3 value (ties to even, saturating at 448, subnormals kept);
  * codes: q = fp32(v / fp32(s g)), rounded to the nearest E2M1 value (ties
    to the even code, saturating at 6), keeping v's sign bit; a block whose
    scale rounds to 0 gets zero codes (with v's sign bit);
  * E2M1 codes packed two per byte, the even element in the low nibble (as
    for MXFP4); scales one E4M3 byte per block, row-major [rows, K / 16].
fp32 steps are written as numpy float32 operations (each rounded once).
"""
from __future__ import annotations

import numpy as np

from . import mx as _mx

BLOCK = 16
F32 = np.float32
G_DIV = F32(6.0 * 448.0)


def global_scale(v: np.ndarray) -> np.float32:
    """fp32(amax / 2688), or 1 for an all-zero tensor."""
    amax = F32(np.max(np.abs(np.asarray(v, F32)), initial=0.0))
    return F32(amax / G_DIV) if amax > 0 else F32(1.0)


def _e4m3_code(s: np.ndarray) -> np.ndarray:
    """Codes of non-negative E4M3 grid values."""
    return _mx._encode_magnitude(np.asarray(s, np.float64), "e4m3").astype(np.uint8)


def quantize(v: np.ndarray, g, axis: int = -1):
    """NVFP4 codes (unpacked, one per byte, sign in bit 3), E4M3 scale
    bytes [.., K/16 ..] for fp32 values v and the tensor's fp32 scale g."""
    g = F32(g)
    v = np.moveaxis(np.asarray(v, F32), axis, -1)
    K = v.shape[-1]
    if K % BLOCK:
        raise ValueError("quantized axis must be a multiple of 16")
    blk = v.reshape(v.shape[:-1] + (K // BLOCK, BLOCK))
    amax = np.abs(blk).max(axis=-1).astype(F32)
    t = (amax / F32(F32(6.0) * g)).astype(F32)
    s = _mx.round_to_grid(t.astype(np.float64), "e4m3")          # exact E4M3 values
    d = (s.astype(F32) * g).astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(d[..., None] > 0, blk / np.where(d > 0, d, F32(1))[..., None], F32(0)).astype(F32)
    r = _mx.round_to_grid(q.astype(np.float64), "e2m1")
    mag = _mx._encode_magnitude(np.abs(r), "e2m1")
    sign = np.signbit(blk).astype(np.int64) << 3
    codes = (mag | sign).reshape(v.shape).astype(np.uint8)
    return np.moveaxis(codes, -1, axis), np.moveaxis(_e4m3_code(s), -1, axis)


def operand_values(codes: np.ndarray, scales: np.ndarray, axis: int = -1) -> np.ndarray:
    """e2m1(code) * e4m3(scale) (exact in fp32 and in bf16): the values an
    NVFP4 operand carries before its tensor scale."""
    c = np.moveaxis(np.asarray(codes), axis, -1)
    s = np.moveaxis(np.asarray(scales), axis, -1)
    val = _mx.element_value(c, "e2m1") * np.repeat(_mx.element_value(s, "e4m3"), BLOCK, axis=-1)
    return np.moveaxis(val.astype(F32), -1, axis)


def dequantize(codes, scales, g, axis: int = -1) -> np.ndarray:
    """fp32(e2m1(code) * e4m3(scale) * g)."""
    return (operand_values(codes, scales, axis) * F32(g)).astype(F32)


def fake_quant(v: np.ndarray, g=None, axis: int = -1) -> np.ndarray:
    """dequantize(quantize(v)) with the tensor scale g (default: v's own)."""
    g = global_scale(v) if g is None else F32(g)
    c, s = quantize(v, g, axis)
    return dequantize(c, s, g, axis)
