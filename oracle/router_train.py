"""Training steps on either side of the routing: the router backward, the
sequence-wise auxiliary balance loss and the aux-loss-free bias update.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this.

[TE-DSV3] Description, DeepSeekV3MoE item: the router is a sigmoid router
with an aux-loss-free bias and grouped top-k; Changes section: an optional
sequence-wise auxiliary loss is listed as a follow-up. The pages give no
formula for any of the three; the readings taken (the DeepSeek-V3 rules)
are:
  * router backward: the expert lists are constants (top-k selection is
    piecewise constant; the bias only takes part in selection, so it gets
    no gradient). The combine weight of slot j is
        w[t, j] = scale * s[t, e_j] / S_t,  S_t = sum_j s[t, e_j],
    so with dw[t, j] = <dOut[t], y[t, j]> (y the expert output row of the
    slot, before weighting) the score gradient of a selected expert is
        ds[t, e_j] = scale / S_t * (dw[t, j] - sum_i dw[t, i] * s[t, e_i] / S_t)
    and zero for every other expert; through the sigmoid
        dlogit = ds * s * (1 - s);
    and through the router GEMM  dx = dlogit . W_r,  dW_r = dlogit^T . x.
  * sequence-wise balance loss over sequences of L consecutive tokens:
        f_i = E / (k L) * #{t in the sequence : expert i selected for t}
        P_i = (1 / L) * sum_t s'[t, i],   s'[t, i] = s[t, i] / sum_m s[t, m]
        loss = alpha * mean over sequences of sum_i f_i P_i
    (f is a constant for the gradient; s' normalizes over all experts);
    its logit gradient (per sequence q of n_seq) is, with
    g_i = alpha / n_seq * f_i / L and Z_t = sum_m s[t, m]:
        dlogit[t, m] += (g_m - sum_i g_i s'[t, i]) / Z_t * s[t, m] (1 - s[t, m]).
  * bias update after a step: b_i <- b_i + gamma * sign(mean_load - load_i),
    load_i = number of (token, slot) pairs routed to expert i in the batch,
    mean_load = T k / E, sign(0) = 0 (an overloaded expert's bias drops).
Everything but the bias update (one fp32 addition) is evaluated in fp64
and rounded once to fp32 at the end.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64
F32 = np.float32


def scores(logits: np.ndarray) -> np.ndarray:
    """sigmoid of the fp32 logits, in fp64."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(logits, F64)))


def combine_weight_grad(dout: np.ndarray, y_sel: np.ndarray) -> np.ndarray:
    """dw[t, j] = <dOut[t], y_sel[t, j]> with y_sel [T, k, H]: the gradient
    of the loss with respect to each combine weight."""
    return np.einsum("th,tjh->tj", np.asarray(dout, F64), np.asarray(y_sel, F64))


def score_grad(s: np.ndarray, idx: np.ndarray, dw: np.ndarray, routed_scale: float) -> np.ndarray:
    """ds [T, E]: the combine-weight gradient pulled back through the
    normalization w = scale * s_sel / sum(s_sel); zero for experts not
    selected."""
    T, E = s.shape
    ds = np.zeros((T, E), F64)
    for t in range(T):
        sel = s[t, idx[t]]
        S = sel.sum()
        inner = float(np.dot(dw[t], sel)) / S
        for j, e in enumerate(idx[t]):
            ds[t, e] += routed_scale / S * (dw[t, j] - inner)
    return ds


def logit_grad_from_scores(ds: np.ndarray, s: np.ndarray) -> np.ndarray:
    return ds * s * (1.0 - s)


def seq_aux_loss(s: np.ndarray, idx: np.ndarray, seq_len: int, alpha: float):
    """Sequence-wise balance loss and its logit gradient [T, E] (fp64)."""
    T, E = s.shape
    k = idx.shape[1]
    if seq_len <= 0 or T % seq_len:
        raise ValueError("T must be a multiple of the sequence length")
    nseq = T // seq_len
    Z = s.sum(axis=1, keepdims=True)
    sp = s / Z
    loss = 0.0
    dl = np.zeros((T, E), F64)
    for q in range(nseq):
        rows = slice(q * seq_len, (q + 1) * seq_len)
        cnt = np.bincount(idx[rows].ravel(), minlength=E).astype(F64)
        f = E / (k * seq_len) * cnt
        P = sp[rows].mean(axis=0)
        loss += float(np.dot(f, P))
        g = alpha / nseq * f / seq_len
        inner = sp[rows] @ g                                   # [L]
        dsq = (g[None, :] - inner[:, None]) / Z[rows]
        dl[rows] += dsq * s[rows] * (1.0 - s[rows])
    return alpha * loss / nseq, dl


def router_backward(x, w_router, logits, idx, dout, y_sel, routed_scale, *, seq_len=0,
                    aux_alpha=0.0):
    """The router backward. x [T, H], w_router [E, H] stored values;
    logits [T, E] fp32 (the forward's); idx [T, k]; dout [T, H]; y_sel
    [T, k, H] the expert output rows of each slot (before weighting).
    Returns dict(dw [T, k], dlogits [T, E], dx [T, H], dw_router [E, H],
    aux_loss) with dw, dlogits, dx, dw_router rounded to fp32."""
    s = scores(logits)
    dw = combine_weight_grad(dout, y_sel)
    dl = logit_grad_from_scores(score_grad(s, idx, dw, routed_scale), s)
    aux = 0.0
    if aux_alpha:
        aux, dl_aux = seq_aux_loss(s, idx, seq_len, aux_alpha)
        dl = dl + dl_aux
    dx = dl @ np.asarray(w_router, F64)
    dwr = dl.T @ np.asarray(x, F64)
    return dict(dw=dw.astype(F32), dlogits=dl.astype(F32), dx=dx.astype(F32),
                dw_router=dwr.astype(F32), aux_loss=F32(aux))


def bias_update(bias: np.ndarray, counts: np.ndarray, k: int, gamma: float) -> np.ndarray:
    """b + gamma * sign(mean_load - load) in fp32 (gamma taken as an fp32
    value; one fp32 addition per expert). The sign compares T k / E with
    the load exactly, in integers: sign(T k - E load)."""
    counts = np.asarray(counts, np.int64)
    E = counts.shape[0]
    total = int(counts.sum())
    sgn = np.sign(total - E * counts).astype(F32)
    return (np.asarray(bias, F32) + F32(gamma) * sgn).astype(F32)
