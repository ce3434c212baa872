"""Pins for the oracle's MX quantizer (E8M0 block scales, E4M3/E2M1 codes).

Pinned against: exhaustive brute force over every finite bf16 bit pattern
(linear search over all codes), textbook round-to-nearest-even boundary
values listed in tests/golden/mx_boundaries.txt, decode tables written out
from the bit-field definitions, and round trips of on-grid values.
"""
import os

import numpy as np
import pytest

from oracle import mx
from tests import brute
from moe_synth import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_boundaries.txt")


def all_finite_bf16() -> np.ndarray:
    bits = np.arange(65536, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    return v[np.isfinite(v)]


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_decode_tables(fmt):
    codes = np.arange(256 if fmt == "e4m3" else 16)
    got = mx.element_value(codes, fmt)
    ref = brute.e4m3_table() if fmt == "e4m3" else brute.e2m1_table()
    finite = ~np.isnan(ref)
    assert np.array_equal(got[finite], ref[finite])
    if fmt == "e4m3":
        assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9
        assert got[0x38] == 1.0 and got[0xFE] == -448.0
    else:
        assert list(got[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_exhaustive_bf16_against_linear_search(fmt):
    """Every finite bf16 value, in blocks of 32 whose amax varies widely."""
    v = all_finite_bf16()
    rng = np.random.default_rng(5)
    v = v[rng.permutation(len(v))]
    n = len(v) // 32 * 32
    blocks = v[:n].reshape(-1, 32)
    codes, scales = mx.quantize(blocks, fmt, axis=-1)
    bc, bs = brute.bf_quantize_blocks(blocks, fmt)
    assert np.array_equal(scales[:, 0], bs)
    assert np.array_equal(codes, bc)
    # every finite code of the format is produced somewhere
    assert len(np.unique(codes)) == (254 if fmt == "e4m3" else 16)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_every_value_in_one_binade_of_scales(fmt):
    """Blocks whose amax sits exactly at 2^emax (scale 2^0): each remaining
    element is checked against the linear search, covering subnormals,
    halfway points and saturation."""
    emax = 8 if fmt == "e4m3" else 2
    maxv = 448.0 if fmt == "e4m3" else 6.0
    table = brute.e4m3_table() if fmt == "e4m3" else brute.e2m1_table()
    fin = table[~np.isnan(table)]
    pos = np.unique(np.abs(fin))
    mids = (pos[1:] + pos[:-1]) / 2
    probes = np.concatenate([pos, mids, mids * (1 + 2 ** -10), mids * (1 - 2 ** -10),
                             [maxv * 1.05, maxv * 1.1, 2.0 ** (emax + 1) * 0.999]])
    probes = np.concatenate([probes, -probes]).astype(np.float32)
    n = -(-len(probes) // 31) * 31
    probes = np.resize(probes, n).reshape(-1, 31)
    blocks = np.concatenate([np.full((probes.shape[0], 1), 2.0 ** emax, np.float32), probes], axis=1)
    codes, scales = mx.quantize(blocks, fmt)
    for b in range(blocks.shape[0]):
        bc, bs = brute.bf_quantize_block(blocks[b], fmt)
        assert scales[b, 0] == bs == 127
        assert np.array_equal(codes[b], bc), (blocks[b], codes[b], bc)


def _load_boundaries():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                fmt, amax, v, want = line.split()
                rows.append((fmt, float(amax), float(v), float(want)))
    return rows


@pytest.mark.parametrize("fmt,amax,v,want", _load_boundaries())
def test_boundary_values(fmt, amax, v, want):
    block = np.zeros((1, 32), np.float32)
    block[0, 0] = amax
    block[0, 1] = v
    c, s = mx.quantize(block, fmt)
    got = mx.dequantize(c, s, fmt)[0, 1]
    assert got == np.float32(want), (fmt, amax, v, got, want)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_on_grid_round_trip_and_axis(fmt):
    rng = np.random.default_rng(0)
    table = brute.e4m3_table() if fmt == "e4m3" else brute.e2m1_table()
    fin = table[~np.isnan(table)]
    grid = rng.choice(fin, (8, 64))
    grid[:, 0] = fin.max()            # pins the block scale to 2^0
    grid[:, 32] = fin.max()
    sc = 2.0 ** rng.integers(-20, 20, (8, 1))
    v = (grid * sc).astype(np.float32)
    assert np.array_equal(mx.fake_quant(v, fmt), v)
    # axis=0 is the transpose of axis=-1
    c0, s0 = mx.quantize(v.T, fmt, axis=0)
    c1, s1 = mx.quantize(v, fmt, axis=-1)
    assert np.array_equal(c0, c1.T) and np.array_equal(s0, s1.T)


def test_zero_block_and_sign():
    z = np.zeros((2, 32), np.float32)
    z[1] = -0.0
    c, s = mx.quantize(z, "e4m3")
    assert (s == 0).all() and (c[0] == 0).all() and (c[1] == 0x80).all()
    assert (mx.dequantize(c, s, "e4m3") == 0).all()


def test_fp4_packing():
    codes = np.arange(32, dtype=np.uint8).reshape(2, 16) % 16
    p = mx.pack_fp4(codes)
    assert p.shape == (2, 8)
    assert p[0, 0] == (0 | (1 << 4)) and p[0, 1] == (2 | (3 << 4))
    assert np.array_equal(mx.unpack_fp4(p), codes)


def test_quantized_error_bound():
    """Relative error of one element is at most half a grid step:
    2^-4 (E4M3) / 2^-2 (E2M1) of the element's binade, below saturation."""
    x = gen.round_to_storage(np.random.default_rng(2).standard_normal((64, 256)), "bf16")
    for fmt, rel in (("e4m3", 2 ** -4), ("e2m1", 2 ** -2)):
        q = mx.fake_quant(x, fmt)
        c, s = mx.quantize(x, fmt)
        scale = np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=1)
        sat = 448.0 if fmt == "e4m3" else 6.0
        ok = np.abs(x) / scale <= sat
        sub = 2.0 ** (-6 if fmt == "e4m3" else 0) * scale
        bound = np.maximum(np.abs(x) * rel, sub * (2 ** -3 if fmt == "e4m3" else 0.5) / 2 * 1.0001)
        assert (np.abs(q - x)[ok] <= bound[ok] * 1.0001).all()
