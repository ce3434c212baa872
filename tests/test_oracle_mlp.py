"""Pins for the oracle's expert MLP, shared expert, combine and the whole
forward.

Pinned against: a dense fp64 evaluation of every expert on every token
combined by a dense [T, E] weight matrix (no permutation at all; the "MoE vs
dense reference" idea of the TE DeepSeekV3Layer test list), the special case
one expert + k = 1 == a dense SwiGLU MLP (torch fp64), the closed form
W1 = [I; I], W2 = I -> silu(x) * x, a constant-row combine, and MX layers
checked against the same dense fp64 evaluation on brute-force-quantized
operands.
"""
import numpy as np
import pytest
import torch

from oracle import mlp, mx, permute as pm, routing as rt
from moe_synth import configs, gen
from tests import brute


def _layer(cfg, seed=0):
    d = gen.host_inputs(cfg, seed)
    shared = (d["w1s"], d["w2s"]) if cfg.n_shared else None
    res = mlp.moe_forward(d["x"], d["w_router"], d["bias"], lambda e: d["w1"][e], lambda e: d["w2"][e],
                          E=cfg.E, n_group=cfg.n_group, topk_group=cfg.topk_group, k=cfg.k,
                          routed_scale=cfg.routed_scale, fmt=cfg.fmt, align=cfg.align,
                          shared_w=shared)
    return d, res


def _dense_w(res, T, E):
    dw = np.zeros((T, E))
    np.put_along_axis(dw, res["idx"].astype(np.int64), res["w"].astype(np.float64), axis=1)
    return dw


@pytest.mark.parametrize("name", ["tiny_fp32", "tiny_fp32_unitx", "mini_fp32"])
def test_forward_equals_dense_fp64(name):
    cfg = configs.get(name)
    d, res = _layer(cfg)
    ref = brute.dense_moe_fp64(d["x"], d["w1"], d["w2"], _dense_w(res, cfg.T, cfg.E))
    assert brute.rel_l2(res["out"], ref) < 2e-6


def test_forward_bf16_values_with_shared_equals_dense_fp64():
    cfg = configs.get("mini_bf16")
    d, res = _layer(cfg)
    ref = brute.dense_moe_fp64(d["x"], d["w1"], d["w2"], _dense_w(res, cfg.T, cfg.E),
                               shared=(d["w1s"], d["w2s"]))
    assert brute.rel_l2(res["out"], ref) < 2e-6
    # the shared expert alone matches a dense fp64 SwiGLU MLP
    ref_s = brute.dense_moe_fp64(d["x"], d["w1s"][None], d["w2s"][None], np.ones((cfg.T, 1)))
    assert brute.rel_l2(res["shared"], ref_s) < 2e-6


def test_single_expert_k1_is_dense_swiglu():
    g = np.random.default_rng(0)
    T, H, F = 37, 64, 48
    x = g.standard_normal((T, H)).astype(np.float32)
    w1 = (g.standard_normal((2 * F, H)) / 8).astype(np.float32)
    w2 = (g.standard_normal((H, F)) / 7).astype(np.float32)
    res = mlp.moe_forward(x, np.ones((1, H), np.float32), np.zeros(1, np.float32),
                          lambda e: w1, lambda e: w2, E=1, n_group=1, topk_group=1, k=1,
                          routed_scale=1.0, fmt="fp32")
    xt = torch.tensor(x, dtype=torch.float64)
    a = xt @ torch.tensor(w1, dtype=torch.float64).T
    ref = (torch.nn.functional.silu(a[:, :F]) * a[:, F:]) @ torch.tensor(w2, dtype=torch.float64).T
    assert (res["w"] == 1.0).all()
    assert brute.rel_l2(res["out"], ref.numpy()) < 2e-6


def test_identity_weights_closed_form():
    g = np.random.default_rng(1)
    T, H, E = 20, 32, 4
    x = g.standard_normal((T, H)).astype(np.float32)
    eye = np.eye(H, dtype=np.float32)
    w1 = np.concatenate([eye, eye])
    res = mlp.moe_forward(x, g.standard_normal((E, H)).astype(np.float32), np.zeros(E, np.float32),
                          lambda e: w1, lambda e: eye, E=E, n_group=2, topk_group=1, k=2,
                          routed_scale=2.5, fmt="fp32")
    x64 = x.astype(np.float64)
    ref = 2.5 * x64 / (1 + np.exp(-x64)) * x64
    assert np.allclose(res["out"], ref, rtol=3e-6, atol=1e-6)


def test_combine_constant_rows():
    T, k, H = 9, 3, 16
    rm = np.arange(T * k).reshape(T, k)
    w = np.random.default_rng(2).uniform(0.1, 1, (T, k)).astype(np.float32)
    w = (w / w.sum(1, keepdims=True) * np.float32(2.5)).astype(np.float32)
    y = np.full((T * k, H), 3.0, np.float32)
    sh = np.full((T, H), 1.0, np.float32)
    out = mlp.combine(y, rm, w, sh)
    assert np.allclose(out, 3.0 * 2.5 + 1.0, rtol=1e-6)


def test_combine_uses_row_map():
    rng = np.random.default_rng(3)
    idx = np.stack([rng.permutation(6)[:2] for _ in range(10)]).astype(np.int32)
    _, _, rm, src = pm.permute_maps(idx, 6, 16)
    y = rng.standard_normal((len(src), 8)).astype(np.float32)
    w = rng.uniform(0, 1, (10, 2)).astype(np.float32)
    out = mlp.combine(y, rm, w)
    ref = np.array([sum(np.float64(w[t, j]) * y[rm[t, j]].astype(np.float64) for j in range(2)) for t in range(10)])
    assert np.allclose(out, ref, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("name", ["mini_mxfp8_decode", "mini_mxfp4"])
def test_mx_forward_against_brute_quantized_dense(name):
    """MX layers: operands are re-quantized by the linear-search quantizer and
    the layer is evaluated densely in fp64; h is quantized per row along F."""
    cfg = configs.get(name)
    T = 12
    d = gen.host_inputs(cfg)
    d["x"] = d["x"][:T]
    fmt = mx.fmt_of(cfg.fmt)

    def bq(v, axis=-1):
        return brute.bf_fake_quant(v, fmt, axis)

    experts = [0, 5]                      # a two-expert layer keeps the brute force quick
    w1 = d["w1"][experts]
    w2 = d["w2"][experts]
    wr = d["w_router"][experts]
    res = mlp.moe_forward(d["x"], wr, d["bias"][experts], lambda e: w1[e], lambda e: w2[e],
                          E=2, n_group=1, topk_group=1, k=1, routed_scale=1.0, fmt=cfg.fmt)
    xq = bq(d["x"])
    w1q = [bq(w) for w in w1]
    w2q = [bq(w) for w in w2]
    out = np.zeros((T, cfg.H))
    for t in range(T):
        e = res["idx"][t, 0]
        a = xq[t] @ w1q[e].T
        F = cfg.F
        h = a[:F] / (1 + np.exp(-a[:F])) * a[F:]
        hq = bq(h.astype(np.float32)[None])[0]
        out[t] = res["w"][t, 0] * (hq @ w2q[e].T)
    # h is quantized from fp32 values on both sides; allow rare code flips
    assert brute.rel_l2(res["out"], out) < 2e-3


def test_forward_subset_of_tokens_matches_full():
    cfg = configs.get("mini_bf16")
    d, full = _layer(cfg)
    toks = [0, 7, 299]
    res = mlp.moe_forward(d["x"], d["w_router"], d["bias"], lambda e: d["w1"][e], lambda e: d["w2"][e],
                          E=cfg.E, n_group=cfg.n_group, topk_group=cfg.topk_group, k=cfg.k,
                          routed_scale=cfg.routed_scale, fmt=cfg.fmt, shared_w=(d["w1s"], d["w2s"]),
                          tokens=toks)
    # BLAS blocking differs with the row count, so equal to fp32 rounding
    assert brute.rel_l2(res["out"], full["out"][toks]) < 1e-6


def test_given_routing_equals_dense_fp64_with_those_experts():
    """The oracle driven by given expert lists (the certified-tie rule): with
    one slot of every token replaced by another expert, the output equals the
    dense fp64 evaluation with the oracle's normalized scores of exactly those
    experts; with its own lists it is bit-identical to the plain run."""
    cfg = configs.get("mini_fp32")
    d, res = _layer(cfg)
    again = mlp.moe_forward(d["x"], d["w_router"], d["bias"], lambda e: d["w1"][e],
                            lambda e: d["w2"][e], E=cfg.E, n_group=cfg.n_group,
                            topk_group=cfg.topk_group, k=cfg.k, routed_scale=cfg.routed_scale,
                            fmt=cfg.fmt, idx=res["idx"])
    assert np.array_equal(again["out"], res["out"]) and np.array_equal(again["w"], res["w"])
    idx = res["idx"].copy()
    for t in range(cfg.T):            # last slot -> the lowest expert not already chosen
        idx[t, -1] = min(set(range(cfg.E)) - set(idx[t].tolist()))
    got = mlp.moe_forward(d["x"], d["w_router"], d["bias"], lambda e: d["w1"][e],
                          lambda e: d["w2"][e], E=cfg.E, n_group=cfg.n_group,
                          topk_group=cfg.topk_group, k=cfg.k, routed_scale=cfg.routed_scale,
                          fmt=cfg.fmt, idx=idx)
    assert np.array_equal(got["idx"], idx)
    s = res["s"].astype(np.float64)
    pick = np.take_along_axis(s, idx.astype(np.int64), axis=1)
    dw = np.zeros((cfg.T, cfg.E))
    np.put_along_axis(dw, idx.astype(np.int64), pick / pick.sum(axis=1, keepdims=True) * cfg.routed_scale,
                      axis=1)
    ref = brute.dense_moe_fp64(d["x"], d["w1"], d["w2"], dw)
    assert brute.rel_l2(got["out"], ref) < 2e-6
    cnt, _, _, _ = brute.bf_permute(idx, cfg.E, 1)
    assert np.array_equal(got["counts"], cnt)


def test_expert_threads_do_not_change_bits():
    """Evaluating experts on several threads gives the same bits as one."""
    cfg = configs.get("mini_mxfp4")
    d = gen.host_inputs(cfg)
    kw = dict(E=cfg.E, n_group=cfg.n_group, topk_group=cfg.topk_group, k=cfg.k,
              routed_scale=cfg.routed_scale, fmt=cfg.fmt)
    one = mlp.moe_forward(d["x"], d["w_router"], d["bias"], lambda e: d["w1"][e],
                          lambda e: d["w2"][e], **kw)
    many = mlp.moe_forward(d["x"], d["w_router"], d["bias"], lambda e: d["w1"][e],
                           lambda e: d["w2"][e], workers=4, **kw)
    assert np.array_equal(one["out"], many["out"])


def test_nvfp4_forward_against_brute_quantized_dense():
    """NVFP4 layer: operands re-quantized by the linear-search NVFP4
    quantizer of tests/test_oracle_nvfp4.py (each weight matrix with its own
    tensor scale, x and h with the layer's fixed ones) and the layer
    evaluated densely in fp64."""
    from tests.test_oracle_nvfp4 import _brute_block
    from oracle import nvfp4
    cfg = configs.get("mini_nvfp4")
    T = 6
    d = gen.host_inputs(cfg)
    d["x"] = d["x"][:T]
    F32 = np.float32

    def bq(v, g):
        v = np.asarray(v, F32)
        out = np.empty(v.shape, np.float64)
        for r in range(v.shape[0]):
            for b in range(v.shape[1] // 16):
                c, s = _brute_block(v[r, 16 * b:16 * b + 16], F32(g))
                vals = brute.e2m1_table()[c] * brute.e4m3_table()[s]
                out[r, 16 * b:16 * b + 16] = (vals.astype(F32) * F32(g)).astype(F32)
        return out

    experts = [0, 5]
    w1 = d["w1"][experts]
    w2 = d["w2"][experts]
    wr = d["w_router"][experts]
    res = mlp.moe_forward(d["x"], wr, d["bias"][experts], lambda e: w1[e], lambda e: w2[e],
                          E=2, n_group=1, topk_group=1, k=1, routed_scale=1.0, fmt=cfg.fmt,
                          act_globals=(cfg.x_global, cfg.h_global))
    xq = bq(d["x"], cfg.x_global)
    w1q = [bq(w, nvfp4.global_scale(w)) for w in w1]
    w2q = [bq(w, nvfp4.global_scale(w)) for w in w2]
    out = np.zeros((T, cfg.H))
    for t in range(T):
        e = res["idx"][t, 0]
        a = xq[t] @ w1q[e].T
        h = a[:cfg.F] / (1 + np.exp(-a[:cfg.F])) * a[cfg.F:]
        hq = bq(h.astype(F32)[None], cfg.h_global)[0]
        out[t] = res["w"][t, 0] * (hq @ w2q[e].T)
    assert brute.rel_l2(res["out"], out) < 2e-3
