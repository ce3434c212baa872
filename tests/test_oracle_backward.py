"""Pins for the oracle's backward (combine, fc2, SwiGLU, fc1, permute, dW).

Pinned against: torch.autograd in fp64 on a dense (permutation-free)
formulation of the layer with routing weights held constant, central finite
differences of an fp64 forward written with numpy, exact zero weight
gradients for experts without rows, and for MX layers an fp64 evaluation of
the same chain on operands re-quantized by the linear-search quantizer.
"""
import numpy as np
import pytest
import torch

from oracle import backward as bw, mlp, routing as rt
from tests import brute


def _tiny(seed=0, T=11, H=32, F=32, E=5, k=2):
    g = np.random.default_rng(seed)
    x = g.standard_normal((T, H)).astype(np.float32)
    w1 = (g.standard_normal((E, 2 * F, H)) / np.sqrt(H)).astype(np.float32)
    w2 = (g.standard_normal((E, H, F)) / np.sqrt(F)).astype(np.float32)
    logits = g.standard_normal((T, E)).astype(np.float32)
    bias = np.zeros(E, np.float32)
    bias[E - 1] = -10.0            # the last expert never gets rows
    idx, w, _, _ = rt.route(logits, bias, 1, 1, k, 1.5)
    dout = g.standard_normal((T, H)).astype(np.float32)
    return x, w1, w2, idx, w, dout


def _autograd(x, w1, w2, idx, w, dout):
    T, k = idx.shape
    E, F2, H = w1.shape
    F = F2 // 2
    X = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    W1 = torch.tensor(w1, dtype=torch.float64, requires_grad=True)
    W2 = torch.tensor(w2, dtype=torch.float64, requires_grad=True)
    dense = torch.zeros((T, E), dtype=torch.float64)
    dense.scatter_(1, torch.tensor(idx, dtype=torch.int64), torch.tensor(w, dtype=torch.float64))
    a = torch.einsum("th,efh->etf", X, W1)
    h = torch.nn.functional.silu(a[..., :F]) * a[..., F:]
    y = torch.einsum("etf,ehf->eth", h, W2)
    out = torch.einsum("te,eth->th", dense, y)
    out.backward(torch.tensor(dout, dtype=torch.float64))
    return X.grad.numpy(), W1.grad.numpy(), W2.grad.numpy(), out.detach().numpy()


def test_matches_fp64_autograd():
    x, w1, w2, idx, w, dout = _tiny()
    res = bw.moe_backward(x, dout, idx, w, lambda e: w1[e], lambda e: w2[e], E=w1.shape[0], fmt="bf16")
    gx, gw1, gw2, _ = _autograd(x, w1, w2, idx, w, dout)
    assert brute.rel_l2(res["dx"], gx) < 2e-6
    for e in range(w1.shape[0] - 1):
        assert brute.rel_l2(res["dw1"][e], gw1[e]) < 2e-6
        assert brute.rel_l2(res["dw2"][e], gw2[e]) < 2e-6


def test_zero_row_expert_has_exact_zero_grads():
    x, w1, w2, idx, w, dout = _tiny()
    assert not (idx == 4).any()
    res = bw.moe_backward(x, dout, idx, w, lambda e: w1[e], lambda e: w2[e], E=5, fmt="mxfp8")
    assert (res["dw1"][4] == 0).all() and (res["dw2"][4] == 0).all()
    assert res["dw1"][4].shape == w1[4].shape


def test_central_finite_differences():
    """<dOut, d out/d theta . v> by central differences of an fp64 numpy
    forward equals <grad, v> for random directions in x, W1 and W2."""
    x, w1, w2, idx, w, dout = _tiny(seed=3, T=6, H=16, F=8, E=3, k=2)
    x, w1, w2, dout = (a.astype(np.float64) for a in (x, w1, w2, dout))
    F = 8

    def fwd(x_, w1_, w2_):
        out = np.zeros_like(x_)
        for t in range(x_.shape[0]):
            for j in range(idx.shape[1]):
                e = idx[t, j]
                a = w1_[e] @ x_[t]
                h = a[:F] / (1 + np.exp(-a[:F])) * a[F:]
                out[t] += float(w[t, j]) * (w2_[e] @ h)
        return out

    res = bw.moe_backward(x.astype(np.float32), dout.astype(np.float32), idx, w,
                          lambda e: w1[e].astype(np.float32), lambda e: w2[e].astype(np.float32),
                          E=3, fmt="bf16")
    g = np.random.default_rng(9)
    eps = 1e-6
    for which in range(3):
        v = [np.zeros_like(x), np.zeros_like(w1), np.zeros_like(w2)]
        v[which] = g.standard_normal(v[which].shape)
        plus = fwd(x + eps * v[0], w1 + eps * v[1], w2 + eps * v[2])
        minus = fwd(x - eps * v[0], w1 - eps * v[1], w2 - eps * v[2])
        fd = float(np.sum(dout * (plus - minus)) / (2 * eps))
        if which == 0:
            an = float(np.sum(res["dx"] * v[0]))
        elif which == 1:
            an = sum(float(np.sum(res["dw1"][e] * v[1][e])) for e in range(3))
        else:
            an = sum(float(np.sum(res["dw2"][e] * v[2][e])) for e in range(3))
        assert abs(fd - an) <= 1e-5 * max(1.0, abs(fd)), (which, fd, an)


def test_mx_backward_against_brute_quantized_chain():
    x, w1, w2, idx, w, dout = _tiny(seed=4, T=40, H=64, F=32, E=2, k=1)
    x = x.astype(np.float32)
    fmt = "e4m3"
    q = lambda v, axis=-1: brute.bf_fake_quant(v, fmt, axis)
    res = bw.moe_backward(x, dout, idx, w, lambda e: w1[e], lambda e: w2[e], E=2, fmt="mxfp8")
    F = 32
    for e in range(2):
        t = np.nonzero(idx[:, 0] == e)[0]
        n = len(t)
        if n == 0:
            continue
        dy = (w[t, 0][:, None].astype(np.float32) * dout[t]).astype(np.float32)
        a = q(x[t]) @ q(w1[e]).T
        g_, u = a[:, :F], a[:, F:]
        sig = 1 / (1 + np.exp(-g_))
        h = g_ * sig * u
        dh = q(dy) @ q(w2[e], axis=0)
        da = np.concatenate([dh * u * sig * (1 + g_ * (1 - sig)), dh * g_ * sig], axis=1)
        dx = q(da.astype(np.float32)) @ q(w1[e], axis=0)
        pad = -(-n // 32) * 32 - n
        P = lambda m: np.concatenate([m, np.zeros((pad, m.shape[1]))]).astype(np.float32)
        dw2 = q(P(dy), axis=0).T @ q(P(h), axis=0)
        dw1 = q(P(da), axis=0).T @ q(P(x[t]), axis=0)
        # intermediates are quantized from fp32 values on both sides: allow
        # rare single-code flips
        assert brute.rel_l2(res["dw2"][e], dw2) < 5e-3
        assert brute.rel_l2(res["dw1"][e], dw1) < 5e-3
        assert brute.rel_l2(res["dx"][t], dx) < 5e-3
