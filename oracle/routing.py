"""Sigmoid router with selection-only bias and grouped top-k.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this.

[TE-DSV3] Description, DeepSeekV3MoE item: "fused sigmoid router with
aux-loss-free bias and grouped top-k". The pages name the steps but print no
formula; the readings taken are:
  * logits = x . W_r^T (plain GEMM, no bias), evaluated in fp64 and rounded
    once to fp32;
  * scores s = sigmoid(logits), evaluated in fp64 and rounded once to fp32;
  * the bias b takes part in *selection only*: sel = fp32(s + b);
  * groups: the E experts split into n_group contiguous groups; a group's
    score is the fp32 sum of its two largest sel values (larger first);
    the topk_group best groups are kept (ties to the lower group index) and
    every other expert's sel becomes -inf;
  * top-k: the k largest masked sel values, in descending order, ties to the
    lower expert index;
  * combine weights: the chosen *unbiased* scores, summed in fp32 in slot
    order, normalized by that sum and then multiplied by the routed scale,
    each step rounded to fp32 (no epsilon).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """[T, H] x [E, H] -> [T, E] fp32, computed in fp64 and rounded once."""
    return (np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T).astype(F32)


def sigmoid_scores(logits: np.ndarray) -> np.ndarray:
    """s = 1 / (1 + exp(-logit)) in fp64, rounded once to fp32."""
    lg = np.asarray(logits, np.float64)
    with np.errstate(over="ignore"):
        return (1.0 / (1.0 + np.exp(-lg))).astype(F32)


def selection_scores(s: np.ndarray, bias: np.ndarray) -> np.ndarray:
    return (np.asarray(s, F32) + np.asarray(bias, F32)).astype(F32)


def group_scores(sel: np.ndarray, n_group: int) -> np.ndarray:
    """[T, E] -> [T, n_group]: sum of the two largest sel values per group."""
    T, E = sel.shape
    g = sel.reshape(T, n_group, E // n_group)
    top = -np.sort(-g, axis=2)
    return (top[:, :, 0] + top[:, :, 1]).astype(F32)


def kept_groups(gscore: np.ndarray, topk_group: int) -> np.ndarray:
    """Indices of the kept groups per token, best first (ties: lower index)."""
    return np.argsort(-gscore, axis=1, kind="stable")[:, :topk_group]


def mask_to_groups(sel: np.ndarray, keep: np.ndarray, n_group: int) -> np.ndarray:
    T, E = sel.shape
    G = E // n_group
    allowed = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(allowed, keep, True, axis=1)
    allowed = np.repeat(allowed, G, axis=1)
    return np.where(allowed, sel, F32(-np.inf)).astype(F32)


def topk_desc(masked: np.ndarray, k: int) -> np.ndarray:
    """k largest per row, descending, ties to the lower index -> int32."""
    return np.argsort(-masked, axis=1, kind="stable")[:, :k].astype(np.int32)


def combine_weights(s: np.ndarray, idx: np.ndarray, routed_scale: float) -> np.ndarray:
    """w[t, j] = fp32(fp32(s[idx] / S) * scale), S = fp32 sum in slot order."""
    picked = np.take_along_axis(np.asarray(s, F32), idx.astype(np.int64), axis=1)
    S = np.zeros(picked.shape[0], dtype=F32)
    for j in range(picked.shape[1]):
        S = (S + picked[:, j]).astype(F32)
    w = (picked / S[:, None]).astype(F32)
    return (w * F32(routed_scale)).astype(F32)


def route(logits: np.ndarray, bias: np.ndarray, n_group: int, topk_group: int,
          k: int, routed_scale: float):
    """Full selection from fp32 logits. Returns (idx [T,k] int32, w [T,k] fp32,
    s [T,E] fp32, sel [T,E] fp32)."""
    s = sigmoid_scores(logits)
    sel = selection_scores(s, bias)
    masked = sel
    if n_group > 1:
        keep = kept_groups(group_scores(sel, n_group), topk_group)
        masked = mask_to_groups(sel, keep, n_group)
    idx = topk_desc(masked, k)
    w = combine_weights(s, idx, routed_scale)
    return idx, w, s, sel
