"""Pins for the oracle's NVFP4 quantizer (oracle.nvfp4).

Pinned against: a brute-force search (the block scale as the nearest of all
E4M3 values by linear scan, each code as the nearest of the 8 E2M1
magnitudes, ties to the even code) on blocks of many magnitudes; exact
round trips of values already on the grid; saturation and zero blocks; the
tensor-scale formula at hand-made amax values; and E2M1 code packing shared
with MXFP4 (low nibble = even element)."""
import numpy as np
import pytest

from oracle import mx, nvfp4
from tests import brute

F32 = np.float32


def _nearest(x: float, vals: np.ndarray) -> int:
    """Index of the nearest value (ties: the even index = even code)."""
    d = np.abs(vals - x)
    best = np.nonzero(d == d.min())[0]
    even = [i for i in best if i % 2 == 0]
    return int(even[0] if even else best[0])


def _brute_block(v: np.ndarray, g: np.float32):
    e4 = brute.e4m3_table()[:127]                 # non-negative finite E4M3 codes 0..126
    amax = F32(np.abs(v).max())
    t = F32(amax / F32(F32(6.0) * g))
    sc = _nearest(float(min(t, 448.0)), e4)
    s = F32(e4[sc])
    codes = []
    mags = np.array(brute.E2M1_VALUES)
    for x in v:
        sign = 8 if np.signbit(x) else 0
        if s == 0:
            codes.append(sign)
            continue
        q = F32(x / F32(s * g))
        codes.append(sign | _nearest(float(min(abs(q), 6.0)), mags))
    return np.array(codes, np.uint8), np.uint8(sc)


@pytest.mark.parametrize("seed", range(4))
def test_quantize_matches_brute_force(seed):
    g_ = np.random.default_rng(seed)
    rows = []
    for _ in range(48):
        rows.append(g_.standard_normal(16) * np.exp2(g_.integers(-12, 10)))
    v = np.array(rows, F32).reshape(-1)
    for gsc in [nvfp4.global_scale(v), F32(2.0 ** -7), F32(0.37)]:
        codes, scales = nvfp4.quantize(v.reshape(12, 64), gsc)
        codes, scales = codes.reshape(-1, 16), scales.reshape(-1)
        for b in range(len(scales)):
            bc, bs = _brute_block(v.reshape(-1, 16)[b], gsc)
            assert bs == scales[b], (b, bs, scales[b])
            assert np.array_equal(bc, codes[b]), b


def test_round_trip_and_saturation():
    g = F32(2.0 ** -5)
    e2 = np.array(brute.E2M1_VALUES)
    # a block whose amax is 6 * s * g with s = 1.5: every grid value times s * g
    s = 1.5
    v = np.array([e2[i % 8] * s * g * (-1) ** i for i in range(16)], F32)
    v[1] = -6 * s * g
    c, sc = nvfp4.quantize(v[None], g)
    assert brute.e4m3_table()[sc[0, 0]] == s
    assert np.array_equal(nvfp4.dequantize(c, sc, g)[0], v)
    # beyond 6 * 448 * g everything saturates to 6 * 448 * g
    big = np.full((1, 16), 1e6, F32)
    c, sc = nvfp4.quantize(big, g)
    assert brute.e4m3_table()[sc[0, 0]] == 448.0 and (c == 7).all()
    assert (nvfp4.dequantize(c, sc, g) == F32(6 * 448) * g).all()
    # zero block: scale 0, codes 0
    c, sc = nvfp4.quantize(np.zeros((2, 32), F32), g)
    assert (c == 0).all() and (sc == 0).all()


def test_global_scale_and_operand_values():
    assert nvfp4.global_scale(np.array([2688.0, -1.0], F32)) == 1.0
    assert nvfp4.global_scale(np.zeros(5, F32)) == 1.0
    assert nvfp4.global_scale(np.array([-5376.0], F32)) == 2.0
    g_ = np.random.default_rng(9)
    v = (g_.standard_normal((8, 64)) * 3).astype(F32)
    gs = nvfp4.global_scale(v)
    c, s = nvfp4.quantize(v, gs)
    # operand values times g are the dequantized values, and the operand
    # values are exact in bf16 (at most 1 + 3 significant bits apiece)
    ov = nvfp4.operand_values(c, s)
    assert np.array_equal((ov * gs).astype(F32), nvfp4.dequantize(c, s, gs))
    bits = ov.view(np.uint32)
    assert (bits & 0xFFFF == 0).all()
    # the error of the format: relative L2 a few percent for normal data
    err = np.linalg.norm(nvfp4.dequantize(c, s, gs) - v) / np.linalg.norm(v)
    assert 0.01 < err < 0.12
    # packing is the MXFP4 one
    assert np.array_equal(mx.unpack_fp4(mx.pack_fp4(c)), c)
