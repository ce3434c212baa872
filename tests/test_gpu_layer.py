"""End-to-end parity of the whole forward (route -> [quantize] -> permute ->
grouped MLP [-> shared expert] -> combine) against the oracle.

* Small and reduced configs: every output element, relative L2 within the
  format's tolerance (fp32 1e-5, bf16 and MXFP8 1e-2, MXFP4 3e-2).
* Full-size configs, in the launch configuration the benchmark times: the
  routing of every token (certified near ties only), counts, and sampled
  output rows the oracle evaluates token by token with weights copied from
  the seeded device generator.
* Special case: one expert, k = 1 is a dense SwiGLU MLP.
"""
import dataclasses

import numpy as np
import pytest
import torch

import mixture_experts_layer_sigmoid_amd as moe
from moe_synth import configs, gen
from oracle import mlp as omlp, routing as rt
from tests.gpu_util import certified_tie_mismatches, dev, device_inputs, host, log, rel_l2

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
                                  "mini_mxfp8_decode", "mini_mxfp4", "mini_skew_mxfp8"])
def test_small_end_to_end(gpu_lib, name):
    cfg = configs.get(name)
    log(f"end-to-end {name}")
    h, fw, out = _forward_small(cfg)
    shared = (h["w1s"], h["w2s"]) if cfg.n_shared else None
    ref = omlp.moe_forward(h["x"], h["w_router"], h["bias"], lambda e: h["w1"][e], lambda e: h["w2"][e],
                           E=cfg.E, n_group=cfg.n_group, topk_group=cfg.topk_group, k=cfg.k,
                           routed_scale=cfg.routed_scale, fmt=cfg.fmt, align=cfg.align, shared_w=shared)
    idx = host(fw.topk_idx)
    nbad, unc = certified_tie_mismatches(ref["sel"], idx, ref["idx"], cfg.n_group, cfg.topk_group)
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
        nbad, unc = certified_tie_mismatches(ref["sel"], host(fw.topk_idx), ref["idx"], cfg.n_group,
                                             cfg.topk_group)
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


@pytest.mark.parametrize("fuse", [False, True])
def test_expert_gemms_run_to_run_identical(gpu_lib, fuse):
    """Repeated fc1 / fc2 launches on the same inputs give the same bits
    (the bf16 layer at full size: 256 experts of mostly one or two 32-row
    blocks, the shape that once read activation rows before their loads had
    landed)."""
    cfg = configs.get("dsv3_bf16_t4096")
    log(f"run-to-run fc1 / fc2 {cfg.name} fuse_shared={fuse}")
    x, wr, b, wts, sh = _full_setup(cfg)
    ew = moe.ExpertWeights.from_dense(wts["w1"], wts["w2"], cfg.fmt)
    sw = moe.ExpertWeights.from_dense(sh["w1s"], sh["w2s"], cfg.fmt)
    del wts
    fw = moe.MoEForward.for_config(cfg, fuse_shared=fuse)
    xd = dev(x, "bf16")
    fw(xd, dev(wr, "bf16"), dev(b), ew, sw)
    torch.cuda.synchronize()
    h0, y0 = fw.h.clone(), fw.y_rows.clone()
    for rep in range(6):
        fw.h.zero_()
        fw.y_rows.zero_()
        fw.experts_fc1(xd, ew, sw=sw)
        fw.experts_fc2(ew, sw=sw)
        torch.cuda.synchronize()
        hb = (fw.h != h0).reshape(fw.h.shape[0], -1).any(dim=1)
        yb = (fw.y_rows != y0).reshape(fw.y_rows.shape[0], -1).any(dim=1)
        assert int(hb.sum()) == 0 and int(yb.sum()) == 0, (rep, int(hb.sum()), int(yb.sum()))


def _full_setup(cfg):
    x = gen.host_x(cfg)
    wr = gen.host_router(cfg)
    b = gen.host_bias(cfg)
    wts = gen.device_expert_weights(cfg, "cuda")
    sh = gen.device_shared_weights(cfg, "cuda") if cfg.n_shared else None
    return x, wr, b, wts, sh


@pytest.mark.parametrize("name,n_sample", [("dsv3_bf16_t4096", 6), ("dsv3_mxfp8_decode_t64", 3),
                                           ("dsv4_mxfp4_t16384", 3)])
def test_full_size_sampled(gpu_lib, name, n_sample):
    cfg = configs.get(name)
    log(f"full-size forward {name}: generating weights on the device")
    x, wr, b, wts, sh = _full_setup(cfg)
    ew = moe.ExpertWeights.from_dense(wts["w1"], wts["w2"], cfg.fmt)
    sw = moe.ExpertWeights.from_dense(sh["w1s"], sh["w2s"], cfg.fmt) if sh else None
    fw = moe.MoEForward.for_config(cfg)
    out = host(fw(dev(x, "bf16"), dev(wr, "bf16"), dev(b), ew, sw))
    torch.cuda.synchronize()
    log(f"  forward done; oracle routing of all {cfg.T} tokens")
    olog = rt.router_logits(x, wr)
    oidx, ow, _, osel = rt.route(olog, b, cfg.n_group, cfg.topk_group, cfg.k, cfg.routed_scale)
    idx = host(fw.topk_idx)
    nbad, unc = certified_tie_mismatches(osel, idx, oidx, cfg.n_group, cfg.topk_group)
    log(f"  routing: {nbad} certified near-tie tokens, {unc} uncertified")
    assert unc == 0 and nbad <= max(2, cfg.T // 1000)
    agree = np.nonzero((idx == oidx).all(axis=1))[0]
    if nbad == 0:
        assert np.array_equal(host(fw.counts), np.bincount(oidx.ravel(), minlength=cfg.E))
    g = np.random.default_rng(11)
    toks = np.unique(np.concatenate([agree[:1], agree[-1:], g.choice(agree, n_sample - 2, replace=False)]))
    log(f"  oracle on sampled tokens {toks.tolist()}")
    w1_host = lambda e: wts["w1"][e].float().cpu().numpy()
    w2_host = lambda e: wts["w2"][e].float().cpu().numpy()
    shared = (sh["w1s"].float().cpu().numpy(), sh["w2s"].float().cpu().numpy()) if sh else None
    ref = omlp.moe_forward(x, wr, b, w1_host, w2_host, E=cfg.E, n_group=cfg.n_group,
                           topk_group=cfg.topk_group, k=cfg.k, routed_scale=cfg.routed_scale,
                           fmt=cfg.fmt, shared_w=shared, logits=olog, tokens=toks)
    err = rel_l2(out[toks], ref["out"])
    log(f"  {name}: sampled rel L2 {err:.3e} (tol {TOL[cfg.fmt]})")
    assert err < TOL[cfg.fmt]
    assert np.isfinite(out).all()
