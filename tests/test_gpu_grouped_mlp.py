"""GPU parity of moe_grouped_mlp_fwd (fc1 + SwiGLU [+ MX h] + fc2) against
the oracle's per-expert MLP, stage by stage: both sides get the same seeded
hidden states, weights and expert-major maps (built by the oracle from a
seeded routing), so only the grouped MLP is under test.

Covers fp32 / bf16 / MXFP8 / MXFP4, row gather through src_row and direct
rows, empty experts, experts longer than one row tile (split into several
tiles), padding rows (must come out zero), the saved fc1 output, and the
shared-expert call shape (E = 1)."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_sigmoid_amd as moe
from moe_synth import configs, gen
from oracle import mlp as omlp, permute as pm
from tests.gpu_util import dev, host, log, rel_l2

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 1e-2, "mxfp8": 1e-2, "mxfp4": 3e-2}
# the saved (unrounded) fc1 output against the oracle's fp32 product
SAVE_TOL = {"fp32": 1e-5, "bf16": 1e-5, "mxfp8": 1e-4, "mxfp4": 1e-4}


def _routing(T, E, k, seed, heavy=0):
    """Seeded distinct-expert routing; expert 0 gets `heavy` extra tokens'
    first slot and the last two experts get none."""
    g = np.random.default_rng(seed)
    idx = np.stack([g.permutation(E - 2)[:k] for _ in range(T)]).astype(np.int32)
    if heavy:
        rows = g.permutation(T)[:heavy]
        for t in rows:
            if 0 not in idx[t]:
                idx[t, 0] = 0
    return idx


def _weights_dev(cfg, h):
    dt = cfg.act_dtype
    w1, w2 = dev(h["w1"], dt), dev(h["w2"], dt)
    return moe.ExpertWeights.from_dense(w1, w2, cfg.fmt)


def _run(cfg, x_d, ew, offsets, src, bound, T, act_save=False, direct_rows=None):
    fmt = cfg.fmt
    f = moe.FMT[fmt]
    act_fmt = moe.FMT["fp32" if fmt == "fp32" else "bf16"]
    if moe.layer.is_mx(fmt):
        src_rows = x_d if direct_rows is None else direct_rows
        a, a_sc = moe.quantize_mx(src_rows, fmt)
    else:
        a, a_sc = (x_d if direct_rows is None else direct_rows), None
    act = x_d.dtype
    y = torch.full((bound, cfg.H), 7.0, dtype=act, device="cuda")
    save = torch.zeros((bound, 2 * cfg.F), dtype=torch.float32, device="cuda") if act_save else None
    ws = torch.empty(max(1, moe.moe_grouped_mlp_workspace(ew.w1.shape[0], cfg.H, cfg.F, bound, f, f)),
                     dtype=torch.uint8, device="cuda")
    off_d = torch.from_numpy(offsets.astype(np.int32)).cuda()
    src_d = None if src is None else torch.from_numpy(src.astype(np.int32)).cuda()
    moe.moe_grouped_mlp_fwd(a, a_sc, f, src_d, ew.w1, ew.w1_sc, ew.w2, ew.w2_sc, f, off_d,
                            ew.w1.shape[0], cfg.H, cfg.F, bound, save, y, act_fmt, ws)
    torch.cuda.synchronize()
    return host(y), (host(save) if act_save else None)


def _oracle_rows(cfg, h, offsets, src, E):
    """y rows (and fc1 outputs) of the oracle in expert-major order."""
    bound = len(src)
    y = np.zeros((bound, cfg.H), np.float32)
    a_all = np.zeros((bound, 2 * cfg.F), np.float32)
    xq = omlp.operand(h["x"], cfg.fmt)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        rows = np.arange(lo, hi)
        live = rows[src[lo:hi] >= 0]
        if len(live) == 0:
            continue
        w1q = omlp.operand(h["w1"][e], cfg.fmt)
        w2q = omlp.operand(h["w2"][e], cfg.fmt)
        a, _, ye = omlp.expert_mlp(xq[src[live]], w1q, w2q, cfg.fmt)
        y[live] = ye
        a_all[live] = a
    return y, a_all


@pytest.mark.parametrize("name,T,k,heavy,align", [
    ("mini_fp32", 200, 3, 0, 1), ("mini_bf16", 600, 2, 420, 1), ("mini_bf16", 37, 8, 0, 32),
    ("mini_mxfp8_decode", 40, 8, 0, 1), ("mini_mxfp8_decode", 500, 3, 380, 16),
    ("mini_mxfp4", 500, 6, 300, 1), ("mini_skew_mxfp8", 300, 6, 290, 32),
    # a segment of 6 / 7 row tiles: groups of 4 row tiles and a partial group
    ("mini_bf16", 1500, 2, 1450, 1), ("mini_mxfp4", 1500, 6, 1450, 1)])
def test_stage_parity(gpu_lib, name, T, k, heavy, align):
    cfg = configs.get(name)
    log(f"grouped MLP stage {name} T={T} k={k} heavy={heavy} align={align}")
    h = gen.host_inputs(cfg)
    g = np.random.default_rng(T)
    x = gen.round_to_storage(g.standard_normal((T, cfg.H)).astype(np.float32), cfg.act_dtype)
    h["x"] = x
    idx = _routing(T, cfg.E, k, T + k, heavy)
    counts, offsets, row_map, src = pm.permute_maps(idx, cfg.E, align)
    assert counts.max() > 256 or heavy == 0
    if heavy > 1000:
        assert counts.max() > 5 * 256 and counts.max() % (4 * 256) != 0
    ew = _weights_dev(cfg, h)
    x_d = dev(x, cfg.act_dtype)
    y, save = _run(cfg, x_d, ew, offsets, src, len(src), T, act_save=True)
    y_ref, a_ref = _oracle_rows(cfg, h, offsets, src, cfg.E)
    used = offsets[-1]
    live = src[:used] >= 0
    err = rel_l2(y[:used][live], y_ref[:used][live])
    log(f"  rel L2 {err:.2e}")
    assert err < TOL[cfg.fmt]
    assert (y[:used][~live] == 0).all(), "padding rows must be zero"
    assert (y[used:] == 7.0).all(), "rows past the segments are not written"
    # the saved fc1 output is the unrounded accumulator: equal to the oracle's
    # fp32 product up to summation order for fp32 and bf16 (1e-5); the MX
    # matrix instructions add each 64-element block product at their own
    # internal precision (1e-4)
    assert rel_l2(save[:used][live], a_ref[:used][live]) < SAVE_TOL[cfg.fmt]


@pytest.mark.parametrize("name,T,k,heavy", [
    ("mini_mxfp8_decode", 16, 8, 0), ("mini_mxfp8_decode", 100, 2, 95), ("mini_bf16", 100, 2, 90),
    ("mini_mxfp4", 120, 2, 100)])
def test_decode_tiles(gpu_lib, name, T, k, heavy):
    """Batches with at most eight rows per expert on average run 64-row
    tiles with a deeper weight ring; an expert with more than 64 rows spans
    several of them."""
    cfg = configs.get(name)
    assert T * k <= 8 * cfg.E
    log(f"grouped MLP decode tiles {name} T={T} k={k} heavy={heavy}")
    h = gen.host_inputs(cfg)
    g = np.random.default_rng(T + 1)
    x = gen.round_to_storage(g.standard_normal((T, cfg.H)).astype(np.float32), cfg.act_dtype)
    h["x"] = x
    idx = _routing(T, cfg.E, k, T + k, heavy)
    counts, offsets, _, src = pm.permute_maps(idx, cfg.E, 1)
    assert heavy == 0 or counts.max() > 64
    ew = _weights_dev(cfg, h)
    y, save = _run(cfg, dev(x, cfg.act_dtype), ew, offsets, src, len(src), T, act_save=True)
    y_ref, a_ref = _oracle_rows(cfg, h, offsets, src, cfg.E)
    err = rel_l2(y, y_ref)
    log(f"  rel L2 {err:.2e}")
    assert err < TOL[cfg.fmt]
    assert rel_l2(save, a_ref) < SAVE_TOL[cfg.fmt]


def test_fallback_tiles_bf16(gpu_lib):
    """Widths that do not fill the kernel's tiles: F = 192 leaves the last fc1
    column tile (128 h columns) half empty, so two of its four waves have no
    columns, and fc2's 384 output columns end in a half-filled 256-column
    tile."""
    cfg = configs.MoEConfig(**{**configs.get("mini_bf16").__dict__, "name": "fallback_bf16",
                               "H": 384, "F": 192, "E": 12, "T": 150, "n_group": 4, "topk_group": 2,
                               "k": 3, "F_shared": 192, "family": "fallback_bf16"})
    log("grouped MLP fallback tiles H=384 F=192")
    h = gen.host_inputs(cfg)
    idx = _routing(cfg.T, cfg.E, 3, 5, heavy=120)
    _, offsets, _, src = pm.permute_maps(idx, cfg.E, 1)
    ew = _weights_dev(cfg, h)
    y, _ = _run(cfg, dev(h["x"], "bf16"), ew, offsets, src, len(src), cfg.T)
    y_ref, _ = _oracle_rows(cfg, h, offsets, src, cfg.E)
    assert rel_l2(y, y_ref) < TOL["bf16"]


@pytest.mark.parametrize("name", ["mini_bf16", "mini_mxfp8_decode", "mini_mxfp4", "mini_fp32"])
def test_direct_rows_equal_gathered_rows(gpu_lib, name):
    cfg = configs.get(name)
    log(f"grouped MLP direct rows vs gather, {name}")
    h = gen.host_inputs(cfg)
    idx = _routing(cfg.T, cfg.E, cfg.k if cfg.k < cfg.E - 2 else 2, 3)
    _, offsets, _, src = pm.permute_maps(idx, cfg.E, 1)
    ew = _weights_dev(cfg, h)
    x_d = dev(h["x"], cfg.act_dtype)
    y1, _ = _run(cfg, x_d, ew, offsets, src, len(src), cfg.T)
    perm = dev(pm.permute_rows(h["x"], src), cfg.act_dtype)
    y2, _ = _run(cfg, x_d, ew, offsets, None, len(src), cfg.T, direct_rows=perm)
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("name", ["mini_bf16", "mini_mxfp8_decode"])
def test_shared_expert_shape(gpu_lib, name):
    """E = 1, offsets {0, T}, no gather: a dense SwiGLU MLP on every token."""
    cfg = configs.get(name)
    log(f"grouped MLP as a shared expert, {name}")
    h = gen.host_inputs(cfg)
    scfg = configs.MoEConfig(**{**cfg.__dict__, "E": 1, "F": cfg.F_shared})
    sh = {"x": h["x"], "w1": h["w1s"][None], "w2": h["w2s"][None]}
    ew = _weights_dev(scfg, sh)
    x_d = dev(h["x"], cfg.act_dtype)
    offsets = np.array([0, cfg.T], np.int32)
    y, _ = _run(scfg, x_d, ew, offsets, None, cfg.T, cfg.T)
    _, _, ref = omlp.expert_mlp(omlp.operand(h["x"], cfg.fmt), omlp.operand(h["w1s"], cfg.fmt),
                                omlp.operand(h["w2s"], cfg.fmt), cfg.fmt)
    assert rel_l2(y, ref) < TOL[cfg.fmt]


@pytest.mark.parametrize("fmt,H,F,E,T,k", [
    ("mxfp8", 2048, 256, 8, 600, 2),     # long K: 16 MX stages, at most one tile per workgroup
    ("bf16", 2048, 256, 8, 600, 2),      # long K: 32 bf16 stages
    ("mxfp8", 512, 512, 64, 4000, 8),    # many tiles per persistent workgroup
    ("bf16", 512, 512, 64, 4000, 8),
    ("mxfp4", 1024, 512, 64, 4000, 8)])
def test_long_k_and_many_tiles(gpu_lib, fmt, H, F, E, T, k):
    """K loops of several full pipeline groups, and more tiles than
    workgroups (every workgroup runs tile after tile); repeated calls must
    agree bit for bit."""
    base = configs.get("mini_bf16")
    cfg = configs.MoEConfig(**{**base.__dict__, "name": f"lk_{fmt}_{H}_{E}", "family": f"lk_{fmt}_{H}_{E}",
                               "H": H, "F": F, "E": E, "T": T, "k": k, "n_group": 1, "topk_group": 1,
                               "fmt": fmt, "F_shared": F})
    log(f"grouped MLP {fmt} H={H} F={F} E={E} T={T} k={k}")
    h = gen.host_inputs(cfg)
    idx = _routing(T, E, k, 17, heavy=0)
    _, offsets, _, src = pm.permute_maps(idx, E, 1)
    ew = _weights_dev(cfg, h)
    x_d = dev(h["x"], cfg.act_dtype)
    y, save = _run(cfg, x_d, ew, offsets, src, len(src), T, act_save=True)
    y_ref, a_ref = _oracle_rows(cfg, h, offsets, src, E)
    # the pipeline is deterministic: repeated calls agree bit for bit
    for _ in range(3):
        y2, save2 = _run(cfg, x_d, ew, offsets, src, len(src), T, act_save=True)
        assert np.array_equal(y, y2) and np.array_equal(save, save2), "run-to-run difference"
    e_a = rel_l2(save, a_ref)
    e_y = rel_l2(y, y_ref)
    log(f"  saved fc1 output {e_a:.2e}, y {e_y:.2e}")
    assert e_a < 1e-4
    assert e_y < TOL[fmt]
