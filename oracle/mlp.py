"""Expert MLPs (fc1 -> SwiGLU -> fc2), shared expert, weighted combine, and
the whole layer forward as a plain per-expert loop.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this.

[TE-DSV3] Description, DeepSeekV3MoE item: experts are GroupedLinear ->
ScaledSwiGLU -> GroupedLinear with an optional shared expert. The
Performance section's "naive" variant — a Python loop of per-expert MLPs —
is the structure followed here. [SGL-NVFP4] Highlights: fc1's weight holds
the w1 (gate) and w3 (up) halves.

Readings taken where the pages are silent:
  * fc1 weight [2F, H]: rows [0, F) gate (the SiLU input), rows [F, 2F) up;
    fc2 weight [H, F]; no biases;
  * SwiGLU: h = silu(g) * u with silu(g) = g * sigmoid(g), in fp32;
  * the routing weight is applied in the combine, not to h (the two agree in
    exact arithmetic since fc2 has no bias);
  * the combine is out[t] = sum_j w[t,j] * y[row(t,j)] in slot order, in
    fp32, plus the shared expert's output with unit weight;
  * MX layers: x is MX-quantized per token along H before fc1, h per row
    along F before fc2; the GEMMs see the dequantized values; expert and
    shared weights are MX-quantized along their contraction axis; the NVFP4
    layer likewise with NVFP4 blocks of 16 (oracle.nvfp4), each expert
    weight matrix with its own tensor scale, x and h with fixed ones;
  * the GEMMs accumulate in fp32; bf16 storage rounding of intermediates is
    not emulated.
"""
from __future__ import annotations

import numpy as np

from . import mx as _mx
from . import nvfp4 as _nv
from . import permute as _perm
from . import routing as _rt

F32 = np.float32


def silu(g: np.ndarray) -> np.ndarray:
    g = np.asarray(g, F32)
    with np.errstate(over="ignore"):
        sig = (F32(1) / (F32(1) + np.exp(-g))).astype(F32)
    return (g * sig).astype(F32)


def swiglu(a: np.ndarray, F: int) -> np.ndarray:
    """a [n, 2F] -> h [n, F] = silu(a[:, :F]) * a[:, F:]."""
    a = np.asarray(a, F32)
    return (silu(a[:, :F]) * a[:, F:]).astype(F32)


def operand(v: np.ndarray, fmt: str, axis: int = -1, g=None) -> np.ndarray:
    """Values a GEMM sees for a stored operand: MX-dequantized for MX
    layers (blocks along the contraction axis), NVFP4-dequantized for the
    NVFP4 layer (tensor scale g; by default the tensor's own, as for a
    weight matrix), unchanged otherwise."""
    if fmt in ("mxfp8", "mxfp4"):
        return _mx.fake_quant(v, _mx.fmt_of(fmt), axis)
    if fmt == "nvfp4":
        return _nv.fake_quant(v, g, axis)
    return np.asarray(v, F32)


def expert_mlp(xq: np.ndarray, w1q: np.ndarray, w2q: np.ndarray, fmt: str, h_global=None):
    """One expert on its rows. xq [n, H], w1q [2F, H], w2q [H, F] are the
    operand values. Returns (a [n, 2F], h [n, F], y [n, H]) in fp32.
    h_global: the tensor scale of h (NVFP4 layer)."""
    F = w1q.shape[0] // 2
    a = (np.asarray(xq, F32) @ np.asarray(w1q, F32).T).astype(F32)
    h = swiglu(a, F)
    hq = operand(h, fmt, axis=-1, g=h_global)
    y = (hq @ np.asarray(w2q, F32).T).astype(F32)
    return a, h, y


def combine(y_rows: np.ndarray, row_map: np.ndarray, w: np.ndarray,
            shared: np.ndarray | None = None) -> np.ndarray:
    """out[t] = sum_j w[t,j] * y_rows[row_map[t,j]] (+ shared[t]), fp32."""
    T, k = row_map.shape
    out = np.zeros((T, y_rows.shape[1]), dtype=F32)
    for j in range(k):
        out = (out + (w[:, j:j + 1].astype(F32) * y_rows[row_map[:, j]].astype(F32))).astype(F32)
    if shared is not None:
        out = (out + np.asarray(shared, F32)).astype(F32)
    return out


def moe_forward(x, w_router, bias, w1_of, w2_of, *, E, n_group, topk_group, k,
                routed_scale, fmt, align=1, shared_w=None, logits=None,
                tokens=None, idx=None, workers=1, act_globals=None):
    """The layer forward.

    x: [T, H] fp32 values of the stored hidden states. w1_of(e) / w2_of(e)
    return expert e's stored weights ([2F, H] / [H, F], fp32 values).
    shared_w: None or (w1s [2Fs, H], w2s [H, Fs]). logits: optional fp32
    router logits to start from (stage-wise mode). tokens: optional subset of
    token indices whose outputs are evaluated (routing and maps always cover
    all T tokens). idx: optional [T, k] expert lists to use instead of the
    oracle's own top-k (where two candidates are within rounding of each
    other several selections are correct; the combine weights are then the
    oracle's normalized scores of those experts). workers: experts evaluated
    concurrently by that many threads (each expert's arithmetic is
    unchanged; only independent experts overlap). act_globals: (g_x, g_h),
    the tensor scales of the hidden states and of h in the NVFP4 layer.
    """
    gx, gh = act_globals if act_globals is not None else (None, None)
    x = np.asarray(x, F32)
    T = x.shape[0]
    if logits is None:
        logits = _rt.router_logits(x, w_router)
    if idx is None:
        idx, w, s, sel = _rt.route(logits, bias, n_group, topk_group, k, routed_scale)
    else:
        idx = np.asarray(idx, np.int32)
        s = _rt.sigmoid_scores(logits)
        sel = _rt.selection_scores(s, bias)
        w = _rt.combine_weights(s, idx, routed_scale)
    counts, offsets, row_map, src_row = _perm.permute_maps(idx, E, align)
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    xq = operand(x[toks], fmt, axis=-1, g=gx)      # per-token quantization
    pos = {int(t): i for i, t in enumerate(toks)}
    sub_idx = idx[toks]

    def one_expert(e):
        tj = np.argwhere(sub_idx == e)             # (token position, slot) in order
        w1q = operand(w1_of(int(e)), fmt, axis=-1)
        w2q = operand(w2_of(int(e)), fmt, axis=-1)
        _, _, ye = expert_mlp(xq[tj[:, 0]], w1q, w2q, fmt, gh)
        return tj, ye

    experts = [int(e) for e in np.unique(sub_idx)]
    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=workers) as ex:
            results = list(ex.map(one_expert, experts))
    else:
        results = [one_expert(e) for e in experts]
    y = {}                                         # (t, j) -> y row
    for tj, ye in results:
        for r, (p, j) in enumerate(tj):
            y[(int(p), int(j))] = ye[r]
    H = x.shape[1]
    y_sub = np.zeros((len(toks) * k, H), dtype=F32)
    rm_sub = np.arange(len(toks) * k).reshape(len(toks), k)
    for p in range(len(toks)):
        for j in range(k):
            y_sub[rm_sub[p, j]] = y[(p, j)]
    ys = None
    if shared_w is not None:
        w1s, w2s = shared_w
        _, _, ys = expert_mlp(xq, operand(w1s, fmt), operand(w2s, fmt), fmt, gh)
    out = combine(y_sub, rm_sub, w[toks], ys)
    return dict(logits=logits, s=s, sel=sel, idx=idx, w=w, counts=counts,
                offsets=offsets, row_map=row_map, src_row=src_row, out=out,
                shared=ys, tokens=toks, pos=pos)
