"""GPU parity of moe_route against the oracle router.

* logits_in path: the same seeded fp32 logits go to both sides, so expert
  indices must match bit for bit and weights within 2 fp32 ulps (both
  evaluate the sigmoid in fp64 and round once).
* GEMM path: logits match the oracle's fp64 logits within fp32 accumulation
  error; expert lists match except certified near ties (candidates whose
  oracle scores lie within what the measured logit difference can move
  them; at most 1e-4 of the tokens, at least one). Covered at small
  sizes and at the full hidden size with few tokens (the router GEMM split
  along H into many chunks) and with 4096 tokens.
"""
import numpy as np
import pytest
import torch

from moe_synth import configs, gen
from oracle import routing as rt
from tests.gpu_util import (certified_tie_mismatches, dev, log, max_tie_tokens, rel_l2, tie_margin,
                            ulp_diff_f32)

pytestmark = pytest.mark.gpu


def _route_dev(gpu_lib, T, H, E, ng, tg, k, scale, bias, logits=None, x=None, w=None, fmt=1):
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lo = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ws = None
    if logits is None:
        ws = torch.empty(max(1, gpu_lib.moe_route_workspace(T, H, E)), dtype=torch.uint8, device="cuda")
    gpu_lib.moe_route(x, fmt, w, bias, logits, T, H, E, ng, tg, k, scale, lo, idx, wt, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), wt.cpu().numpy(), lo.cpu().numpy()


@pytest.mark.parametrize("T,E,ng,tg,k,scale", [
    (64, 16, 4, 2, 4, 1.0), (4096, 256, 8, 4, 8, 2.5), (333, 384, 1, 1, 6, 1.0),
    (77, 256, 1, 1, 6, 1.0), (5, 512, 64, 8, 16, 1.5), (50, 2, 1, 1, 2, 1.0), (1, 24, 6, 3, 5, 1.0)])
def test_logits_in_bit_exact(gpu_lib, T, E, ng, tg, k, scale):
    log(f"route logits_in T={T} E={E} groups={ng}/{tg} k={k}")
    g = np.random.default_rng(T + E)
    logits = (g.standard_normal((T, E)) * g.choice([0.01, 1.0, 6.0])).astype(np.float32)
    logits[0, : min(E, 8)] = 0.0          # exact ties
    bias = g.uniform(-0.05, 0.05, E).astype(np.float32)
    idx, w, lo = _route_dev(gpu_lib, T, 0, E, ng, tg, k, scale, dev(bias), logits=dev(logits))
    oidx, ow, _, _ = rt.route(logits, bias, ng, tg, k, scale)
    assert np.array_equal(lo, logits)
    assert np.array_equal(idx, oidx)
    assert ulp_diff_f32(w, ow).max() <= 2


@pytest.mark.parametrize("name", ["tiny_fp32", "tiny_fp32_unitx", "mini_fp32", "mini_bf16", "mini_mxfp4",
                                  "mini_skew_mxfp8"])
def test_gemm_path_small(gpu_lib, name):
    cfg = configs.get(name)
    log(f"route with router GEMM, {name}")
    x = gen.host_x(cfg)
    wr = gen.host_router(cfg)
    b = gen.host_bias(cfg)
    idx, w, lo = _route_dev(gpu_lib, cfg.T, cfg.H, cfg.E, cfg.n_group, cfg.topk_group, cfg.k,
                            cfg.routed_scale, dev(b), x=dev(x, cfg.act_dtype), w=dev(wr, cfg.act_dtype),
                            fmt=0 if cfg.act_dtype == "fp32" else 1)
    olog = rt.router_logits(x, wr)
    assert rel_l2(lo, olog) < 1e-6
    oidx, ow, _, osel = rt.route(olog, b, cfg.n_group, cfg.topk_group, cfg.k, cfg.routed_scale)
    nbad, unc, _ = certified_tie_mismatches(osel, idx, oidx, cfg.n_group, cfg.topk_group,
                                            margin=tie_margin(lo, olog))
    assert unc == 0 and nbad <= max_tie_tokens(cfg.T, cfg.bias_kind)
    same = (idx == oidx).all(axis=1)
    assert rel_l2(w[same], ow[same]) < 1e-5


@pytest.mark.parametrize("name", ["dsv3_bf16_t4096", "dsv4_mxfp4_t16384", "dsv4_skew_mxfp8_t8192"])
def test_gemm_path_full_size(gpu_lib, name):
    cfg = configs.get(name)
    log(f"route with router GEMM, full size {name}")
    x = gen.host_x(cfg)
    wr = gen.host_router(cfg)
    b = gen.host_bias(cfg)
    idx, w, lo = _route_dev(gpu_lib, cfg.T, cfg.H, cfg.E, cfg.n_group, cfg.topk_group, cfg.k,
                            cfg.routed_scale, dev(b), x=dev(x, "bf16"), w=dev(wr, "bf16"))
    olog = rt.router_logits(x, wr)
    assert rel_l2(lo, olog) < 1e-6
    oidx, ow, _, osel = rt.route(olog, b, cfg.n_group, cfg.topk_group, cfg.k, cfg.routed_scale)
    margin = tie_margin(lo, olog)
    nbad, unc, bad = certified_tie_mismatches(osel, idx, oidx, cfg.n_group, cfg.topk_group,
                                              margin=margin)
    log(f"  {name}: margin {margin:.2e}; {nbad} mismatched tokens of {cfg.T} {bad.tolist()}, "
        f"{unc} uncertified")
    assert unc == 0 and nbad <= max_tie_tokens(cfg.T, cfg.bias_kind)
    same = (idx == oidx).all(axis=1)
    assert rel_l2(w[same], ow[same]) < 1e-5
    # the same call again gives the same bits
    idx2, w2, lo2 = _route_dev(gpu_lib, cfg.T, cfg.H, cfg.E, cfg.n_group, cfg.topk_group, cfg.k,
                               cfg.routed_scale, dev(b), x=dev(x, "bf16"), w=dev(wr, "bf16"))
    assert np.array_equal(lo.view(np.uint32), lo2.view(np.uint32))
    assert np.array_equal(idx, idx2) and np.array_equal(w.view(np.uint32), w2.view(np.uint32))


@pytest.mark.parametrize("name", ["dsv3_mxfp8_decode_t64", "dsv3_bf16_t4096", "dsv4_skew_mxfp8_t8192"])
def test_gemm_path_full_hidden(gpu_lib, name):
    cfg = configs.get(name)
    log(f"route with router GEMM at full hidden size, {name} (H split {gpu_lib.moe_route_workspace(cfg.T, cfg.H, cfg.E) // (4 * cfg.T * cfg.E)} ways)")
    x = gen.host_x(cfg)
    wr = gen.host_router(cfg)
    b = gen.host_bias(cfg)
    idx, w, lo = _route_dev(gpu_lib, cfg.T, cfg.H, cfg.E, cfg.n_group, cfg.topk_group, cfg.k,
                            cfg.routed_scale, dev(b), x=dev(x, "bf16"), w=dev(wr, "bf16"))
    olog = rt.router_logits(x, wr)
    assert rel_l2(lo, olog) < 1e-6
    oidx, ow, _, osel = rt.route(olog, b, cfg.n_group, cfg.topk_group, cfg.k, cfg.routed_scale)
    nbad, unc, _ = certified_tie_mismatches(osel, idx, oidx, cfg.n_group, cfg.topk_group,
                                            margin=tie_margin(lo, olog))
    assert unc == 0 and nbad <= max_tie_tokens(cfg.T, cfg.bias_kind)
    same = (idx == oidx).all(axis=1)
    assert ulp_diff_f32(w[same], ow[same]).max() <= 64     # fp32 logits vs fp64 logits
