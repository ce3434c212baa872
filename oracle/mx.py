"""MX block quantization (E4M3 / E2M1 elements, E8M0 block scales).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this.

What the pages give: the MXFP8 recipe quantizes the received (dispatched)
rows before the grouped GEMMs ([TE-DSV3] Performance section, "Where the time
goes" table, MXFP8 quantization row) and the 4-bit W4A4 MoE of [SGL-NVFP4]
(Modifications section). The element/scale formats are one E8M0 scale per 32
consecutive elements along the contraction axis with E4M3 or E2M1 elements.

Readings taken where the pages are silent (OCP MX v1.0 conventions):
  * block scale exponent  e = floor(log2(amax)) - emax_elem, clamped to
    [-127, 127]; scale byte = e + 127; emax_elem = 8 (E4M3), 2 (E2M1);
  * elements: nearest value of the element grid to v / 2^e, ties to the even
    code, saturating to +-max (448 for E4M3, 6 for E2M1); no inf/NaN output;
  * amax == 0: scale byte 0; the element codes keep the sign bit of v;
  * every element code carries the sign bit of its input (so a negative value
    that rounds to zero gives the negative-zero code);
  * E2M1 codes are packed two per byte, the even element in the low nibble.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32

# element formats: (exponent bias, mantissa bits, max finite value, emax)
FORMATS = {
    "e4m3": dict(bias=7, mbits=3, maxval=448.0, emax=8, bits=8),
    "e2m1": dict(bias=1, mbits=1, maxval=6.0, emax=2, bits=4),
}


def element_value(code: np.ndarray, fmt: str) -> np.ndarray:
    """Decode element codes to fp64 values (plain bit-field definition)."""
    f = FORMATS[fmt]
    code = np.asarray(code, dtype=np.int64)
    nb = f["bits"]
    sign = np.where((code >> (nb - 1)) & 1, -1.0, 1.0)
    exp = (code >> f["mbits"]) & ((1 << (nb - 1 - f["mbits"])) - 1)
    man = code & ((1 << f["mbits"]) - 1)
    frac = man / float(1 << f["mbits"])
    sub = frac * 2.0 ** (1 - f["bias"])
    nrm = (1.0 + frac) * 2.0 ** (exp - f["bias"])
    return sign * np.where(exp == 0, sub, nrm)


def _encode_magnitude(r: np.ndarray, fmt: str) -> np.ndarray:
    """Code bits (without sign) of representable non-negative values r."""
    f = FORMATS[fmt]
    min_normal = 2.0 ** (1 - f["bias"])
    out = np.zeros(r.shape, dtype=np.int64)
    sub = r < min_normal
    # subnormal: r = man * 2^(1 - bias - mbits)
    out[sub] = np.rint(r[sub] / 2.0 ** (1 - f["bias"] - f["mbits"])).astype(np.int64)
    nz = ~sub
    if np.any(nz):
        m, ex = np.frexp(r[nz])          # r = m * 2^ex, m in [0.5, 1)
        p = ex - 1                       # floor(log2 r)
        man = np.rint((r[nz] / 2.0 ** p - 1.0) * (1 << f["mbits"])).astype(np.int64)
        out[nz] = ((p + f["bias"]) << f["mbits"]) | man
    return out


def round_to_grid(y: np.ndarray, fmt: str) -> np.ndarray:
    """Nearest element-grid value to y (fp64), ties to even code, saturated."""
    f = FORMATS[fmt]
    a = np.abs(y)
    min_normal = 2.0 ** (1 - f["bias"])
    # quantum (spacing of the grid) at |y|
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(np.where(a > 0, a, 1.0))
    p = np.maximum(ex - 1, int(np.log2(min_normal)))
    q = 2.0 ** (p - f["mbits"])
    r = np.round(a / q) * q              # numpy rounds halves to even
    r = np.minimum(r, f["maxval"])
    return np.copysign(r, y)


def quantize(v: np.ndarray, fmt: str, axis: int = -1):
    """MX-quantize fp32 values along `axis` in blocks of 32.

    Returns (codes uint8 with the shape of v, scales uint8 with v's shape but
    axis length / 32). E2M1 codes are returned unpacked (one per byte)."""
    f = FORMATS[fmt]
    v = np.asarray(v, dtype=np.float32)
    v = np.moveaxis(v, axis, -1)
    K = v.shape[-1]
    if K % BLOCK:
        raise ValueError("quantized axis must be a multiple of 32")
    blk = v.reshape(v.shape[:-1] + (K // BLOCK, BLOCK)).astype(np.float64)
    amax = np.abs(blk).max(axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    e = np.clip(ex - 1 - f["emax"], -127, 127)
    scale_byte = np.where(amax > 0, e + 127, 0).astype(np.int64)
    y = blk / np.exp2(scale_byte - 127.0)[..., None]
    r = round_to_grid(y, fmt)
    mag = _encode_magnitude(np.abs(r), fmt)
    sign = (np.signbit(blk).astype(np.int64)) << (f["bits"] - 1)
    codes = (mag | sign).reshape(v.shape).astype(np.uint8)
    codes = np.moveaxis(codes, -1, axis)
    scales = np.moveaxis(scale_byte.astype(np.uint8), -1, axis)
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray, fmt: str, axis: int = -1) -> np.ndarray:
    """fp32 values code_value * 2^(scale-127), blocks of 32 along `axis`."""
    c = np.moveaxis(np.asarray(codes), axis, -1)
    s = np.moveaxis(np.asarray(scales), axis, -1)
    val = element_value(c, fmt)
    sc = np.exp2(np.repeat(s.astype(np.float64), BLOCK, axis=-1) - 127.0)
    out = (val * sc).astype(np.float32)
    return np.moveaxis(out, -1, axis)


def fake_quant(v: np.ndarray, fmt: str, axis: int = -1) -> np.ndarray:
    """dequantize(quantize(v)) — the values an MX GEMM operand carries."""
    c, s = quantize(v, fmt, axis)
    return dequantize(c, s, fmt, axis)


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """Two E2M1 codes per byte along the last axis, even element low."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 15) | ((c[..., 1::2] & 15) << 4)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def fmt_of(layer_fmt: str) -> str:
    """Element format of an MX layer format name."""
    return {"mxfp8": "e4m3", "mxfp4": "e2m1"}[layer_fmt]
