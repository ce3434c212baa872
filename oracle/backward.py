"""Backward of the routed expert path (combine, fc2, SwiGLU, fc1, permute),
with per-expert weight gradients.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this.

[TE-DSV3] Performance section, "Where the time goes" table: the fused
grouped MLP runs "dGLU bwd" and "wgrad" in MXFP8. The pages give no formula;
the readings taken are:
  * routing weights are constants (no router or bias gradient);
  * quantizers pass gradients straight through;
  * every backward GEMM operand is MX-quantized along that GEMM's
    contraction axis: dY and W2 along H for dH; dA and W1 along 2F for dX;
    dY, h, dA and x along the rows of the expert segment (blocks of 32 rows
    of the segment padded with zero rows to a multiple of 32) for dW;
  * h and A for the backward are recomputed in fp32 from the forward inputs.

Chain (fp32 throughout):
  dY_row   = w[t,j] * dOut[t]
  dH       = dY . W2                       [n, F]
  dgate    = dH * up * sig(g) * (1 + g * (1 - sig(g)))
  dup      = dH * silu(g)
  dX_row   = [dgate, dup] . W1              [n, H]
  dX[t]    = sum_j dX_row[row(t, j)]        (slot order)
  dW2_e    = dY_e^T . h_e                   [H, F]
  dW1_e    = dA_e^T . x_e                   [2F, H]
Experts with no rows get exactly zero weight gradients.
"""
from __future__ import annotations

import numpy as np

from . import mlp as _mlp

F32 = np.float32
ROW_BLOCK = 32


def _pad_rows(a: np.ndarray, mult: int) -> np.ndarray:
    n = a.shape[0]
    m = (n + mult - 1) // mult * mult
    if m == n:
        return a
    return np.concatenate([a, np.zeros((m - n,) + a.shape[1:], dtype=a.dtype)])


def expert_backward(x_rows, dy_rows, w1, w2, fmt):
    """One expert. x_rows [n, H] stored inputs, dy_rows [n, H] weighted
    upstream gradients (fp32), w1 [2F, H], w2 [H, F] stored weights.
    Returns (dx_rows [n, H], dw1 [2F, H], dw2 [H, F]) in fp32."""
    F = w1.shape[0] // 2
    n = x_rows.shape[0]
    xq = _mlp.operand(x_rows, fmt, axis=-1)
    a = (xq @ _mlp.operand(w1, fmt, axis=-1).T).astype(F32)
    g, u = a[:, :F], a[:, F:]
    h = _mlp.swiglu(a, F)
    with np.errstate(over="ignore"):
        sig = (F32(1) / (F32(1) + np.exp(-g))).astype(F32)
    dh = (_mlp.operand(dy_rows, fmt, axis=-1) @ _mlp.operand(w2, fmt, axis=0)).astype(F32)
    dgate = (dh * u * sig * (F32(1) + g * (F32(1) - sig))).astype(F32)
    dup = (dh * (g * sig)).astype(F32)
    da = np.concatenate([dgate, dup], axis=1).astype(F32)
    dx = (_mlp.operand(da, fmt, axis=-1) @ _mlp.operand(w1, fmt, axis=0)).astype(F32)
    # weight gradients contract over the rows of the (padded) segment
    dyp = _mlp.operand(_pad_rows(np.asarray(dy_rows, F32), ROW_BLOCK), fmt, axis=0)
    hp = _mlp.operand(_pad_rows(h, ROW_BLOCK), fmt, axis=0)
    dap = _mlp.operand(_pad_rows(da, ROW_BLOCK), fmt, axis=0)
    xp = _mlp.operand(_pad_rows(np.asarray(x_rows, F32), ROW_BLOCK), fmt, axis=0)
    dw2 = (dyp.T @ hp).astype(F32)
    dw1 = (dap.T @ xp).astype(F32)
    assert dx.shape == (n, w1.shape[1])
    return dx, dw1, dw2


def moe_backward(x, dout, idx, w, w1_of, w2_of, *, E, fmt, experts=None):
    """x [T, H], dout [T, H] stored values; idx, w the routing of the
    forward. Returns dict(dx [T, H], dw1 {e: [2F, H]}, dw2 {e: [H, F]}).
    `experts` restricts the weight gradients to a subset (dx is complete
    only when every expert is included)."""
    x = np.asarray(x, F32)
    dout = np.asarray(dout, F32)
    T, k = idx.shape
    H = x.shape[1]
    dx_rows = np.zeros((T, k, H), dtype=F32)
    dw1, dw2 = {}, {}
    todo = range(E) if experts is None else experts
    for e in todo:
        tj = np.argwhere(idx == e)
        w1, w2 = w1_of(e), w2_of(e)
        if len(tj) == 0:
            dw1[e] = np.zeros(w1.shape, F32)
            dw2[e] = np.zeros(w2.shape, F32)
            continue
        t, j = tj[:, 0], tj[:, 1]
        dy = (w[t, j][:, None].astype(F32) * dout[t]).astype(F32)
        dxe, dw1[e], dw2[e] = expert_backward(x[t], dy, w1, w2, fmt)
        dx_rows[t, j] = dxe
    dx = np.zeros((T, H), dtype=F32)
    for j in range(k):
        dx = (dx + dx_rows[:, j]).astype(F32)
    return dict(dx=dx, dw1=dw1, dw2=dw2)
