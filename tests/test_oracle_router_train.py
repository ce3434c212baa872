"""Pins for the oracle's router backward, sequence-wise balance loss and
bias update (oracle.router_train).

Pinned against: torch autograd in fp64 (a library routine) of the layer's
routed output and of the balance loss, each as a function of the router
inputs, with the expert lists held fixed; central finite differences of the
oracle's own loss; closed forms of the balance loss (uniform scores give
alpha for any selection; one expert taking every token gives alpha * E * p);
and the sign rule of the bias update on hand-made loads."""
import numpy as np
import pytest
import torch

from oracle import router_train as rtr, routing as rt


def _case(T=24, H=32, E=16, k=4, ng=4, tg=2, seed=0):
    g = np.random.default_rng(seed)
    x = g.standard_normal((T, H)).astype(np.float32)
    wr = (g.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32)
    b = g.uniform(-0.1, 0.1, E).astype(np.float32)
    logits = rt.router_logits(x, wr)
    idx, w, s, sel = rt.route(logits, b, ng, tg, k, 2.5)
    y_sel = g.standard_normal((T, k, H)).astype(np.float32)
    dout = g.standard_normal((T, H)).astype(np.float32)
    return x, wr, logits, idx, y_sel, dout


def _torch_out(x, wr, idx, y_sel, scale):
    """sum_j w[t, j] * y_sel[t, j] with w from sigmoid scores of x . W_r^T,
    the expert lists fixed (fp64)."""
    lg = x @ wr.T
    s = torch.sigmoid(lg)
    sel = torch.gather(s, 1, torch.tensor(idx, dtype=torch.int64))
    w = scale * sel / sel.sum(dim=1, keepdim=True)
    return (w[:, :, None] * torch.tensor(y_sel, dtype=torch.float64)).sum(dim=1)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_router_backward_matches_autograd(seed):
    x, wr, logits, idx, y_sel, dout = _case(seed=seed)
    res = rtr.router_backward(x, wr, logits, idx, dout, y_sel, 2.5)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(wr, dtype=torch.float64, requires_grad=True)
    out = _torch_out(xt, wt, idx, y_sel, 2.5)
    loss = (out * torch.tensor(dout, dtype=torch.float64)).sum()
    gx, gw = torch.autograd.grad(loss, (xt, wt))
    rel = lambda a, b: np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel(res["dx"], gx.numpy()) < 1e-6
    assert rel(res["dw_router"], gw.numpy()) < 1e-6
    # unselected experts get no logit gradient
    mask = np.zeros(res["dlogits"].shape, bool)
    np.put_along_axis(mask, idx.astype(np.int64), True, axis=1)
    assert (res["dlogits"][~mask] == 0).all()


def test_combine_weight_gradient_sums_to_zero_direction():
    """Scaling every selected score of a token by the same factor leaves its
    weights unchanged, so the score gradient is orthogonal to s on the
    selected experts: sum_j ds[t, e_j] * s[t, e_j] == 0."""
    x, wr, logits, idx, y_sel, dout = _case(seed=5)
    s = rtr.scores(logits)
    ds = rtr.score_grad(s, idx, rtr.combine_weight_grad(dout, y_sel), 2.5)
    dots = (ds * s).sum(axis=1)
    assert np.abs(dots).max() < 1e-12 * np.abs(ds).max() * s.shape[1] + 1e-15


@pytest.mark.parametrize("seq_len", [6, 24])
def test_aux_loss_gradient_matches_autograd(seq_len):
    x, wr, logits, idx, y_sel, dout = _case(seed=3)
    loss, dl = rtr.seq_aux_loss(rtr.scores(logits), idx, seq_len, 1e-2)
    lt = torch.tensor(logits, dtype=torch.float64, requires_grad=True)
    s = torch.sigmoid(lt)
    sp = s / s.sum(dim=1, keepdim=True)
    T, E = logits.shape
    k = idx.shape[1]
    total = 0
    for q in range(T // seq_len):
        r = slice(q * seq_len, (q + 1) * seq_len)
        cnt = torch.tensor(np.bincount(idx[r].ravel(), minlength=E), dtype=torch.float64)
        total = total + (E / (k * seq_len) * cnt * sp[r].mean(dim=0)).sum()
    lref = 1e-2 * total / (T // seq_len)
    (g,) = torch.autograd.grad(lref, (lt,))
    assert abs(loss - lref.item()) < 1e-12
    assert np.abs(dl - g.numpy()).max() < 1e-12


def test_aux_loss_finite_differences():
    """The oracle's own loss against its gradient, central differences."""
    x, wr, logits, idx, y_sel, dout = _case(seed=4)
    lg = logits.astype(np.float64)
    _, dl = rtr.seq_aux_loss(rtr.scores(lg), idx, 12, 0.1)
    h = 1e-6
    for t, e in [(0, 0), (3, 5), (17, 11), (23, 15)]:
        p, m = lg.copy(), lg.copy()
        p[t, e] += h
        m[t, e] -= h
        fd = (rtr.seq_aux_loss(rtr.scores(p), idx, 12, 0.1)[0]
              - rtr.seq_aux_loss(rtr.scores(m), idx, 12, 0.1)[0]) / (2 * h)
        assert abs(fd - dl[t, e]) < 1e-8


def test_aux_loss_closed_forms():
    T, E, k, L = 32, 8, 2, 16
    g = np.random.default_rng(0)
    idx = np.stack([g.permutation(E)[:k] for _ in range(T)])
    # uniform scores: every s' is 1/E and sum_i f_i = E, so the loss is alpha
    loss, _ = rtr.seq_aux_loss(np.full((T, E), 0.3), idx, L, 0.7)
    assert abs(loss - 0.7) < 1e-12
    # two experts, top-1, every token picks expert 0 with s'[t, 0] = p:
    # f_0 = 2, f_1 = 0, loss = alpha * 2 * p
    p = 0.8
    s = np.tile([p, 1 - p], (T, 1)) * 0.5
    loss, _ = rtr.seq_aux_loss(s, np.zeros((T, 1), np.int64), L, 0.3)
    assert abs(loss - 0.3 * 2 * p) < 1e-12


def test_bias_update_sign_rule():
    E, k = 8, 2
    counts = np.array([4, 4, 4, 4, 4, 4, 4, 4])        # balanced: mean 4
    b = np.linspace(-0.1, 0.1, E).astype(np.float32)
    assert np.array_equal(rtr.bias_update(b, counts, k, 1e-3), b)
    counts = np.array([10, 0, 4, 4, 3, 5, 4, 2])
    nb = rtr.bias_update(b, counts, k, 1e-3)
    g = np.float32(1e-3)
    for e in range(E):
        want = b[e] - g if counts[e] > 4 else (b[e] + g if counts[e] < 4 else b[e])
        assert nb[e] == np.float32(want), e
