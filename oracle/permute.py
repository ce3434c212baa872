"""Expert-major permutation maps, row gather and the summing un-permute.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this.

[TE-DSV3] Performance section, "Where the time goes" table, local permute
row: a staging buffer is laid out expert-major with zero-filled padding
("dup"), and the expert outputs are reduced back to token order ("reduce").
Readings: rows of one expert are in (token, slot) lexicographic order; each
expert segment is padded to a multiple of `align`; padding rows carry no
token (source -1) and zero bytes; rows past the last segment, up to the
buffer bound T*k + E*(align-1), are padding as well.
"""
from __future__ import annotations

import numpy as np


def rows_bound(T: int, k: int, E: int, align: int) -> int:
    return T * k + E * (align - 1)


def permute_maps(idx: np.ndarray, E: int, align: int):
    """Returns counts [E], offsets [E+1], row_map [T,k], src_row [bound]."""
    idx = np.asarray(idx)
    T, k = idx.shape
    counts = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            counts[idx[t, j]] += 1
    padded = (counts + align - 1) // align * align
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    row_map = np.zeros((T, k), dtype=np.int64)
    nxt = offsets[:-1].copy()
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            row_map[t, j] = nxt[e]
            nxt[e] += 1
    src_row = np.full(rows_bound(T, k, E, align), -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            src_row[row_map[t, j]] = t
    return (counts.astype(np.int32), offsets.astype(np.int32),
            row_map.astype(np.int32), src_row.astype(np.int32))


def permute_rows(rows: np.ndarray, src_row: np.ndarray) -> np.ndarray:
    """Gather token rows into expert-major order; padding rows are zero."""
    rows = np.asarray(rows)
    out = np.zeros((len(src_row),) + rows.shape[1:], dtype=rows.dtype)
    live = src_row >= 0
    out[live] = rows[src_row[live]]
    return out


def unpermute_sum(perm_rows: np.ndarray, row_map: np.ndarray) -> np.ndarray:
    """out[t] = sum_j perm_rows[row_map[t, j]], fp32, in slot order."""
    T, k = row_map.shape
    out = np.zeros((T,) + perm_rows.shape[1:], dtype=np.float32)
    for j in range(k):
        out = (out + perm_rows[row_map[:, j]].astype(np.float32)).astype(np.float32)
    return out
