"""End-to-end parity of the whole forward (route -> [quantize] -> permute ->
grouped MLP [-> shared expert] -> combine) against the oracle.

* Small and reduced configs: every output element, relative L2 within the
  format's tolerance (fp32 1e-5, bf16 and MXFP8 1e-2, MXFP4 3e-2).
* Full-size configs, in the launch configuration the benchmark times: the
  routing of every token (certified near ties only, with the margin derived
  from the measured logit error), counts and maps bit for bit against the
  oracle's permute of the GPU's expert lists, the combine weights, and the
  output of many tokens, every element: all 64 decode tokens; 256 tokens of
  the 4096-token batch that together reach every expert; 64 tokens of the
  MXFP4 batch and of the expert-parallel share (8 experts x 4096 rows);
  tokens of the skewed batch that include rows of its busiest expert. Tie tokens are always among them, checked against the oracle
  driven by the GPU's expert lists. Weights are copied from the seeded
  device generator.
* Repeated expert GEMM launches give identical bits (bf16, MXFP8, MXFP4).
* Special case: one expert, k = 1 is a dense SwiGLU MLP.
"""
import dataclasses

import numpy as np
import pytest
import torch

import mixture_experts_layer_sigmoid_amd as moe
from moe_synth import configs, gen
from oracle import mlp as omlp, routing as rt
from oracle import permute as pm
from tests.gpu_util import (certified_tie_mismatches, dev, device_inputs, host, log, max_tie_tokens,
                            oracle_workers, rel_l2, tie_margin, ulp_diff_f32)

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 1e-2, "mxfp8": 1e-2, "mxfp4": 3e-2}


def _bits(t):
    """Raw storage of a device tensor (bf16 as int16, codes as bytes)."""
    if isinstance(t, np.ndarray):
        return t
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).cpu().numpy()


def _forward_small(cfg):
    h, d = device_inputs(cfg)
    fw = moe.MoEForward.for_config(cfg)
    ew = moe.ExpertWeights.from_dense(d["w1"], d["w2"], cfg.fmt)
    sw = moe.ExpertWeights.from_dense(d["w1s"], d["w2s"], cfg.fmt) if cfg.n_shared else None
    out = fw(d["x"], d["w_router"], d["bias"], ew, sw)
    torch.cuda.synchronize()
    return h, fw, host(out)


@pytest.mark.parametrize("name", ["tiny_fp32", "tiny_fp32_unitx", "mini_fp32", "mini_bf16",
                                  "mini_mxfp8_decode", "mini_mxfp4", "mini_skew_mxfp8",
                                  "mini_ep8_mxfp8"])
def test_small_end_to_end(gpu_lib, name):
    cfg = configs.get(name)
    log(f"end-to-end {name}")
    h, fw, out = _forward_small(cfg)
    shared = (h["w1s"], h["w2s"]) if cfg.n_shared else None
    ref = omlp.moe_forward(h["x"], h["w_router"], h["bias"], lambda e: h["w1"][e], lambda e: h["w2"][e],
                           E=cfg.E, n_group=cfg.n_group, topk_group=cfg.topk_group, k=cfg.k,
                           routed_scale=cfg.routed_scale, fmt=cfg.fmt, align=cfg.align, shared_w=shared)
    idx = host(fw.topk_idx)
    nbad, unc, _ = certified_tie_mismatches(ref["sel"], idx, ref["idx"], cfg.n_group, cfg.topk_group,
                                            margin=0.0)
    assert unc == 0 and nbad == 0, (nbad, unc)
    assert np.array_equal(host(fw.counts), ref["counts"])
    assert np.array_equal(host(fw.offsets), ref["offsets"])
    assert np.array_equal(host(fw.row_map), ref["row_map"])
    assert np.array_equal(host(fw.src_row)[: fw.bound], ref["src_row"])
    err = rel_l2(out, ref["out"])
    log(f"  {name}: rel L2 {err:.3e} (tol {TOL[cfg.fmt]})")
    assert err < TOL[cfg.fmt]


@pytest.mark.parametrize("name", ["mini_bf16", "mini_mxfp8_decode", "mini_mxfp4"])
def test_empty_and_single_token_batches(gpu_lib, name):
    """T = 0 runs every stage as a no-op and returns an empty output; T = 1
    matches the oracle."""
    base = configs.get(name)
    for T in (0, 1):
        cfg = dataclasses.replace(base, T=T)
        log(f"forward {name} T={T}")
        h, fw, out = _forward_small(cfg)
        assert out.shape == (T, cfg.H)
        if T == 0:
            continue
        shared = (h["w1s"], h["w2s"]) if cfg.n_shared else None
        ref = omlp.moe_forward(h["x"], h["w_router"], h["bias"], lambda e: h["w1"][e],
                               lambda e: h["w2"][e], E=cfg.E, n_group=cfg.n_group,
                               topk_group=cfg.topk_group, k=cfg.k, routed_scale=cfg.routed_scale,
                               fmt=cfg.fmt, align=cfg.align, shared_w=shared)
        nbad, unc, _ = certified_tie_mismatches(ref["sel"], host(fw.topk_idx), ref["idx"],
                                                cfg.n_group, cfg.topk_group, margin=0.0)
        assert unc == 0 and nbad == 0, (nbad, unc)
        assert rel_l2(out, ref["out"]) < TOL[cfg.fmt]


def test_single_expert_k1_is_dense_swiglu(gpu_lib):
    g = np.random.default_rng(0)
    T, H, F = 100, 256, 128
    x = gen.round_to_storage(g.standard_normal((T, H)), "bf16")
    w1 = gen.round_to_storage(g.standard_normal((1, 2 * F, H)) / 16, "bf16")
    w2 = gen.round_to_storage(g.standard_normal((1, H, F)) / 11, "bf16")
    fw = moe.MoEForward(T=T, H=H, F=F, E=1, n_group=1, topk_group=1, k=1, routed_scale=1.0, fmt="bf16")
    out = fw(dev(x, "bf16"), dev(np.ones((1, H), np.float32), "bf16"), dev(np.zeros(1, np.float32)),
             moe.ExpertWeights.from_dense(dev(w1, "bf16"), dev(w2, "bf16"), "bf16"))
    torch.cuda.synchronize()
    xt = torch.tensor(x, dtype=torch.float64)
    a = xt @ torch.tensor(w1[0], dtype=torch.float64).T
    ref = (torch.nn.functional.silu(a[:, :F]) * a[:, F:]) @ torch.tensor(w2[0], dtype=torch.float64).T
    assert (host(fw.topk_w) == 1.0).all()
    assert rel_l2(host(out), ref.numpy()) < 1e-2


@pytest.mark.parametrize("name,T", [("mini_bf16", None), ("mini_bf16", 5),
                                    ("mini_mxfp8_decode", None), ("mini_mxfp8_decode", 16),
                                    ("dsv3_bf16_t4096", None),
                                    ("dsv3_mxfp8_decode_t64", None)])
def test_shared_fold_matches_separate(gpu_lib, name, T):
    """The shared expert inside the routed fc1 / fc2 launches computes every
    row with the arithmetic of the separate launches: routed and shared rows,
    their MX codes and the layer output agree bit for bit. T = 5 leaves most
    of the dense expert's eight row parts empty."""
    cfg = configs.get(name)
    if T is not None:
        cfg = dataclasses.replace(cfg, T=T)
    log(f"shared-expert fold {cfg.name} T={cfg.T}")
    if cfg.H > 1024:      # full-size weights come from the device generator
        x, wr, b, wts, sh = _full_setup(cfg)
        d = dict(x=dev(x, "bf16"), w_router=dev(wr, "bf16"), bias=dev(b), w1=wts["w1"],
                 w2=wts["w2"], w1s=sh["w1s"], w2s=sh["w2s"])
    else:
        _, d = device_inputs(cfg)
    ew = moe.ExpertWeights.from_dense(d["w1"], d["w2"], cfg.fmt)
    sw = moe.ExpertWeights.from_dense(d["w1s"], d["w2s"], cfg.fmt)
    runs = []
    for fuse in (True, False):
        fw = moe.MoEForward.for_config(cfg, fuse_shared=fuse)
        assert fw.fuse_shared == fuse
        out = host(fw(d["x"], d["w_router"], d["bias"], ew, sw))
        torch.cuda.synchronize()
        nb, T = fw.bound, cfg.T
        hs, hs_sc = (fw.h[nb:nb + T], fw.h_sc) if fuse else (fw.hs[:T], fw.hs_sc)
        parts = [out, fw.y_rows[:nb], fw.y_shared, fw.h[:nb], hs]
        if fw.h_sc is not None:
            parts += [fw.h_sc[:nb], fw.h_sc[nb:nb + T] if fuse else fw.hs_sc[:T]]
        runs.append([_bits(p) for p in parts])
    names = ["out", "routed y", "shared y", "routed h", "shared h", "routed h scales",
             "shared h scales"]
    for nm, a, b in zip(names, runs[0], runs[1]):
        assert np.array_equal(a, b), nm


@pytest.mark.parametrize("name,fuse", [("dsv3_bf16_t4096", False), ("dsv3_bf16_t4096", True),
                                       ("dsv3_mxfp8_decode_t64", True), ("dsv4_mxfp4_t16384", False),
                                       ("dsv3_ep8_mxfp8_t4096", False)])
def test_expert_gemms_run_to_run_identical(gpu_lib, name, fuse):
    """Repeated fc1 / fc2 launches on the same inputs give the same bits: the
    bf16 layer at full size (256 experts of mostly one or two 32-row blocks,
    the shape that once read activation rows before their loads had landed),
    the MXFP8 decode batch (64-row tiles, deep weight ring), the MXFP4
    batch (block-scaled 4-bit operands, h MX-encoded in the epilogue) and the
    expert-parallel share (MXFP8, full 256-row tiles over 4096-row experts)."""
    cfg = configs.get(name)
    log(f"run-to-run fc1 / fc2 {cfg.name} fuse_shared={fuse}")
    x, wr, b, wts, sh = _full_setup(cfg)
    ew = moe.ExpertWeights.from_dense(wts["w1"], wts["w2"], cfg.fmt)
    sw = moe.ExpertWeights.from_dense(sh["w1s"], sh["w2s"], cfg.fmt) if sh else None
    del wts
    fw = moe.MoEForward.for_config(cfg, fuse_shared=fuse)
    xd = dev(x, "bf16")
    fw(xd, dev(wr, "bf16"), dev(b), ew, sw)
    torch.cuda.synchronize()
    # the rows the GEMMs write: every expert segment and, when folded, the
    # shared expert's rows from `bound` on (the slack rows between the last
    # segment and `bound` that the aligned permute reserves are never written)
    nrow, nb = int(fw.offsets[-1]), fw.bound
    full = [fw.h, fw.y_rows] + ([fw.h_sc] if fw.h_sc is not None else [])
    bufs = [t[:nrow] for t in full]
    if fuse and sh is not None:
        bufs += [t[nb:nb + cfg.T] for t in full]
    first = [t.clone() for t in bufs]
    for rep in range(6):
        for t in full:
            t.zero_()
        fw.experts_fc1(xd, ew, sw=sw)
        fw.experts_fc2(ew, sw=sw)
        torch.cuda.synchronize()
        diff = [int((a != b).reshape(a.shape[0], -1).any(dim=1).sum()) for a, b in zip(bufs, first)]
        assert sum(diff) == 0, (rep, diff)


def _full_setup(cfg):
    x = gen.host_x(cfg)
    wr = gen.host_router(cfg)
    b = gen.host_bias(cfg)
    wts = gen.device_expert_weights(cfg, "cuda")
    sh = gen.device_shared_weights(cfg, "cuda") if cfg.n_shared else None
    return x, wr, b, wts, sh


def _covering_tokens(idx, E, n, seed):
    """n tokens (or all, if fewer) that together route to every expert that
    has rows: one token per expert, rarest experts first, then random
    fill."""
    g = np.random.default_rng(seed)
    chosen = set()
    counts = np.bincount(idx.ravel(), minlength=E)
    for e in np.argsort(counts, kind="stable"):
        if counts[e] == 0 or any(e in idx[t] for t in chosen):
            continue
        chosen.add(int(g.choice(np.nonzero((idx == e).any(axis=1))[0])))
    rest = np.setdiff1d(np.arange(idx.shape[0]), np.array(sorted(chosen), dtype=np.int64))
    fill = max(0, n - len(chosen))
    chosen |= set(int(t) for t in g.choice(rest, min(fill, len(rest)), replace=False))
    return np.array(sorted(chosen), dtype=np.int64)


def _sample_tokens(name, idx, E, T):
    g = np.random.default_rng(11)
    if name == "dsv3_mxfp8_decode_t64":
        return np.arange(T)                                   # every token
    if name == "dsv3_bf16_t4096":
        return _covering_tokens(idx, E, 256, 12)              # every expert reached
    if name in ("dsv4_mxfp4_t16384", "dsv3_ep8_mxfp8_t4096"):
        return np.sort(g.choice(T, 64, replace=False))
    # skewed batch: 8 tokens of the busiest expert, 4 of a mid-size one, 4 more
    counts = np.bincount(idx.ravel(), minlength=E)
    heavy = int(np.argmax(counts))
    nz = np.nonzero(counts)[0]
    mid = int(nz[np.argsort(counts[nz])[len(nz) // 2]])
    pick = lambda e, n: g.choice(np.nonzero((idx == e).any(axis=1))[0], n, replace=False)
    toks = np.concatenate([pick(heavy, 8), pick(mid, 4), g.choice(T, 4, replace=False)])
    return np.unique(toks)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["dsv3_mxfp8_decode_t64", "dsv3_bf16_t4096", "dsv4_mxfp4_t16384",
                                  "dsv4_skew_mxfp8_t8192", "dsv3_ep8_mxfp8_t4096"])
def test_full_size_forward(gpu_lib, name):
    cfg = configs.get(name)
    log(f"full-size forward {name}: generating weights on the device")
    x, wr, b, wts, sh = _full_setup(cfg)
    ew = moe.ExpertWeights.from_dense(wts["w1"], wts["w2"], cfg.fmt)
    sw = moe.ExpertWeights.from_dense(sh["w1s"], sh["w2s"], cfg.fmt) if sh else None
    fw = moe.MoEForward.for_config(cfg, keep_logits=True)
    out = host(fw(dev(x, "bf16"), dev(wr, "bf16"), dev(b), ew, sw))
    torch.cuda.synchronize()
    del ew, sw
    log(f"  forward done; oracle routing of all {cfg.T} tokens")
    olog = rt.router_logits(x, wr)
    lo = host(fw.logits)
    assert rel_l2(lo, olog) < 1e-6
    margin = tie_margin(lo, olog)
    oidx, ow, os_, osel = rt.route(olog, b, cfg.n_group, cfg.topk_group, cfg.k, cfg.routed_scale)
    idx = host(fw.topk_idx)
    nbad, unc, bad = certified_tie_mismatches(osel, idx, oidx, cfg.n_group, cfg.topk_group,
                                              margin=margin)
    log(f"  routing: max |logit diff| gives margin {margin:.2e}; {nbad} certified near-tie tokens "
        f"{bad.tolist()}, {unc} uncertified")
    assert unc == 0 and nbad <= max_tie_tokens(cfg.T, cfg.bias_kind)
    # maps bit for bit against the oracle's permute of the GPU's expert lists
    counts, offsets, row_map, src = pm.permute_maps(idx, cfg.E, cfg.align)
    assert np.array_equal(host(fw.counts), counts)
    assert np.array_equal(host(fw.offsets), offsets)
    assert np.array_equal(host(fw.row_map), row_map)
    assert np.array_equal(host(fw.src_row)[: fw.bound], src)
    # combine weights: the oracle's normalized scores of those experts
    # (fp32 logits on the GPU, fp64 in the oracle)
    assert ulp_diff_f32(host(fw.topk_w), rt.combine_weights(os_, idx, cfg.routed_scale)).max() <= 64
    toks = np.union1d(_sample_tokens(name, idx, cfg.E, cfg.T), bad)
    nexp = len(np.unique(idx[toks]))
    log(f"  oracle on {len(toks)} tokens ({nexp} experts, {oracle_workers()} threads)")
    lock = __import__("threading").Lock()

    def w_host(name_, e):
        with lock:
            u = wts[name_][e].view(torch.int16).cpu().numpy()
        return gen.bf16_bits_to_f32(u.view(np.uint16))
    shared = (host(sh["w1s"]), host(sh["w2s"])) if sh else None
    ref = omlp.moe_forward(x, wr, b, lambda e: w_host("w1", e), lambda e: w_host("w2", e), E=cfg.E,
                           n_group=cfg.n_group, topk_group=cfg.topk_group, k=cfg.k,
                           routed_scale=cfg.routed_scale, fmt=cfg.fmt, shared_w=shared, logits=olog,
                           tokens=toks, idx=idx, workers=oracle_workers())
    got = out[toks]
    err = rel_l2(got, ref["out"])
    per_tok = [rel_l2(got[i], ref["out"][i]) for i in range(len(toks))]
    worst = int(np.argmax(per_tok))
    log(f"  {name}: {len(toks)} tokens, every element: rel L2 {err:.3e} (tol {TOL[cfg.fmt]}); "
        f"worst token {int(toks[worst])} {per_tok[worst]:.3e}")
    assert err < TOL[cfg.fmt]
    assert np.isfinite(out).all()
