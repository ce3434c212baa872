"""Brute-force and fp64 references used to pin the oracle.

Each routine here reaches the same result as an oracle function by a
different route (linear search instead of arithmetic rounding, tuple sorts
instead of array sorts, dense evaluation over all experts instead of the
per-expert loop, fp64 autograd instead of the hand-written chain rule), so a
slip in either shows up as a mismatch.
"""
from __future__ import annotations

import math

import numpy as np
import torch

E4M3_MAX = 448.0
E2M1_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def e4m3_table():
    """Decoded value of every E4M3 code (OCP FP8: 1-4-3, bias 7, no inf,
    S.1111.111 is NaN)."""
    vals = []
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 7
        if e == 15 and m == 7:
            vals.append(float("nan"))
        elif e == 0:
            vals.append(s * m * 2.0 ** -9)
        else:
            vals.append(s * (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


def e2m1_table():
    return np.array([(-1.0 if c & 8 else 1.0) * E2M1_VALUES[c & 7] for c in range(16)])


def bf_scale_exponent(amax: float, emax: int) -> int:
    """Smallest-search for e with 2^emax <= amax / 2^e < 2^(emax+1)."""
    for e in range(-160, 160):
        r = amax / 2.0 ** e
        if 2.0 ** emax <= r < 2.0 ** (emax + 1):
            return e
    raise AssertionError("no exponent found")


def bf_quantize_blocks(blocks: np.ndarray, fmt: str):
    """Blocks [n, 32] -> (codes [n, 32], scale bytes [n]) by search: the
    scale exponent by scanning e for 2^emax <= amax / 2^e < 2^(emax+1), each
    code by comparing against every finite code of the same sign (nearest
    value, ties to the even code)."""
    table = e4m3_table() if fmt == "e4m3" else e2m1_table()
    emax = 8 if fmt == "e4m3" else 2
    nbits = 8 if fmt == "e4m3" else 4
    b = np.asarray(blocks, np.float64)
    amax = np.abs(b).max(axis=1)
    e = np.full(len(b), 999, dtype=np.int64)
    for cand in range(-160, 160):
        r = amax / 2.0 ** cand
        hit = (2.0 ** emax <= r) & (r < 2.0 ** (emax + 1)) & (e == 999)
        e[hit] = cand
    e = np.where(amax == 0, -127, np.clip(e, -127, 127))
    assert (e != 999).all()
    y = b / np.exp2(e.astype(np.float64))[:, None]
    neg = np.signbit(b)
    codes = np.zeros(b.shape, dtype=np.int64)
    best = np.full(b.shape, np.inf)
    for c in range(1 << nbits):
        if np.isnan(table[c]):
            continue
        same = neg == bool((c >> (nbits - 1)) & 1)
        d = np.abs(y - table[c])
        better = same & ((d < best) | ((d == best) & (c % 2 == 0)))
        codes[better] = c
        best[better] = d[better]
    return codes.astype(np.uint8), (e + 127).astype(np.int64)


def bf_quantize_block(block: np.ndarray, fmt: str):
    c, s = bf_quantize_blocks(np.asarray(block)[None], fmt)
    return c[0], int(s[0])


def bf_fake_quant(v: np.ndarray, fmt: str, axis: int = -1) -> np.ndarray:
    """Values after quantize + dequantize via the brute-force quantizer."""
    table = e4m3_table() if fmt == "e4m3" else e2m1_table()
    v = np.moveaxis(np.asarray(v, np.float32), axis, -1)
    blocks = v.reshape(-1, 32)
    c, s = bf_quantize_blocks(blocks, fmt)
    out = table[c] * np.exp2(s.astype(np.float64) - 127)[:, None]
    return np.moveaxis(out.reshape(v.shape), -1, axis)


def bf_route(logits: np.ndarray, bias: np.ndarray, n_group: int, topk_group: int,
             k: int, routed_scale: float):
    """Selection with Python loops and tuple sorts."""
    T, E = logits.shape
    G = E // n_group
    idx = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float32)
    for t in range(T):
        s = [np.float32(1.0 / (1.0 + math.exp(-float(logits[t, e])))) for e in range(E)]
        sel = [np.float32(s[e] + np.float32(bias[e])) for e in range(E)]
        if n_group > 1:
            gsc = []
            for q in range(n_group):
                mem = sorted((sel[e] for e in range(q * G, (q + 1) * G)), reverse=True)
                gsc.append((np.float32(mem[0] + mem[1]), q))
            kept = [q for _, q in sorted(gsc, key=lambda p: (-p[0], p[1]))[:topk_group]]
            cand = [e for q in kept for e in range(q * G, (q + 1) * G)]
        else:
            cand = list(range(E))
        pick = sorted(cand, key=lambda e: (-sel[e], e))[:k]
        idx[t] = pick
        tot = np.float32(0)
        for e in pick:
            tot = np.float32(tot + s[e])
        for j, e in enumerate(pick):
            w[t, j] = np.float32(np.float32(s[e] / tot) * np.float32(routed_scale))
    return idx, w


def bf_permute(idx: np.ndarray, E: int, align: int):
    """Maps from one sort of (expert, token, slot) triples."""
    T, k = idx.shape
    trip = sorted((int(idx[t, j]), t, j) for t in range(T) for j in range(k))
    counts = [0] * E
    for e, _, _ in trip:
        counts[e] += 1
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + -(-counts[e] // align) * align)
    row_map = np.zeros((T, k), dtype=np.int32)
    seen = [0] * E
    for e, t, j in trip:
        row_map[t, j] = offsets[e] + seen[e]
        seen[e] += 1
    bound = T * k + E * (align - 1)
    src = np.full(bound, -1, dtype=np.int32)
    for e, t, j in trip:
        src[row_map[t, j]] = t
    return np.array(counts, np.int32), np.array(offsets, np.int32), row_map, src


def dense_moe_fp64(x, w1, w2, dense_w, shared=None):
    """Every expert on every token in fp64, combined with a dense [T, E]
    weight matrix (zero off the chosen experts): no permutation at all."""
    xt = torch.as_tensor(np.asarray(x, np.float64))
    W1 = torch.as_tensor(np.asarray(w1, np.float64))
    W2 = torch.as_tensor(np.asarray(w2, np.float64))
    F = W1.shape[1] // 2
    a = torch.einsum("th,efh->etf", xt, W1)
    h = torch.nn.functional.silu(a[..., :F]) * a[..., F:]
    y = torch.einsum("etf,ehf->eth", h, W2)
    out = torch.einsum("te,eth->th", torch.as_tensor(np.asarray(dense_w, np.float64)), y)
    if shared is not None:
        w1s, w2s = (torch.as_tensor(np.asarray(a_, np.float64)) for a_ in shared)
        Fs = w1s.shape[0] // 2
        as_ = xt @ w1s.T
        out = out + (torch.nn.functional.silu(as_[:, :Fs]) * as_[:, Fs:]) @ w2s.T
    return out.numpy()


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))
