"""GPU parity of the MXFP8 backward of the routed expert path against the
oracle (oracle.backward), stage by stage and end to end.

Stages get the same seeded synthetic inputs on both sides:
* combine backward (dY rows) and the summing un-permute: bit-exact;
* the transposed (axis 1) weight quantization and the segment-transposed
  activation quantization (rows / gathered tokens): bit-exact codes and
  scales; the recomputed-SwiGLU mode within rounding of silu;
* the grouped weight-gradient GEMM on ragged segments (empty, shorter than
  one 128-row stage, several stages): relative L2 within the MXFP8 bar.
End to end: the reduced skewed config (every expert, zero-row experts give
exact zeros) and the full-size one on its busiest expert (all 8192 rows), a
mid-size and a light expert plus the zero-row experts, with a property
check of the un-permute on sampled tokens and a repeat of the whole
backward that must give the same bits."""
import dataclasses

import numpy as np
import pytest
import torch

import mixture_experts_layer_sigmoid_amd as moe
from moe_synth import configs, gen
from oracle import backward as obw, mx as omx, permute as pm, routing as rt
from tests.gpu_util import (certified_tie_mismatches, dev, device_inputs, host, log, max_tie_tokens,
                            rel_l2, tie_margin)

pytestmark = pytest.mark.gpu

TOL = 1e-2
I32 = dict(dtype=torch.int32, device="cuda")


def _bf16(a):
    return gen.round_to_storage(np.asarray(a, np.float32), "bf16")


def _maps(T, E, k, align, seed, n_empty=3):
    """Seeded routing with distinct experts per token, the last n_empty
    experts unused and expert 0 heavy (several 128-row stages)."""
    g = np.random.default_rng(seed)
    idx = np.stack([g.permutation(E - n_empty)[:k] for _ in range(T)]).astype(np.int32)
    for t in g.permutation(T)[: (2 * T) // 3]:
        if 0 not in idx[t]:
            idx[t, 0] = 0
    counts, offsets, row_map, src = pm.permute_maps(idx, E, align)
    return idx, counts, offsets, row_map, src


def test_combine_bwd_and_unpermute(gpu_lib):
    T, E, k, H = 211, 16, 4, 384
    log(f"combine backward / unpermute T={T} E={E} k={k} H={H}")
    idx, counts, offsets, row_map, src = _maps(T, E, k, 32, 1)
    bound = len(src)
    g = np.random.default_rng(2)
    dout = _bf16(g.standard_normal((T, H)))
    w = g.uniform(0.05, 1.0, (T, k)).astype(np.float32)
    dy = torch.full((bound, H), 3.0, dtype=torch.bfloat16, device="cuda")
    dyf = torch.full((bound, H), 3.0, dtype=torch.float32, device="cuda")
    dyq = torch.full((bound, H), 3, dtype=torch.uint8, device="cuda")
    dys = torch.full((bound, H // 32), 3, dtype=torch.uint8, device="cuda")
    row_w = torch.full((bound,), 3.0, dtype=torch.float32, device="cuda")
    rm, sr = torch.from_numpy(row_map.astype(np.int32)).cuda(), torch.from_numpy(src.astype(np.int32)).cuda()
    d_dout, d_w = dev(dout, "bf16"), dev(w)
    moe.moe_combine_bwd(d_dout, moe.MOE_BF16, rm, sr, d_w, T, k, H, bound, dy, moe.MOE_BF16, None, None)
    moe.moe_combine_bwd(d_dout, moe.MOE_BF16, rm, sr, d_w, T, k, H, bound, dyf, moe.MOE_F32, None, None)
    moe.moe_combine_bwd(d_dout, moe.MOE_BF16, rm, sr, d_w, T, k, H, bound, dyq, moe.MOE_MXFP8_E4M3, dys,
                        row_w)
    torch.cuda.synchronize()
    ref = np.zeros((bound, H), np.float32)
    ref_w = np.zeros(bound, np.float32)
    for t in range(T):
        for j in range(k):
            ref[row_map[t, j]] = w[t, j] * dout[t]
            ref_w[row_map[t, j]] = w[t, j]
    assert np.array_equal(host(dy), _bf16(ref))
    assert np.array_equal(host(dyf), ref)
    assert np.array_equal(host(row_w), ref_w)
    qc, qs = omx.quantize(ref, "e4m3", axis=-1)
    assert np.array_equal(host(dyq), qc) and np.array_equal(host(dys), qs)
    # un-permute of random expert rows: fp32 sums in slot order, bf16 out
    rows = _bf16(g.standard_normal((bound, H)))
    dx = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    moe.moe_unpermute(dev(rows, "bf16"), moe.MOE_BF16, rm, T, k, H, dx, moe.MOE_BF16)
    torch.cuda.synchronize()
    assert np.array_equal(host(dx), _bf16(pm.unpermute_sum(rows, row_map)))
    dxf = torch.empty((T, H), dtype=torch.float32, device="cuda")
    moe.moe_unpermute(dev(rows, "bf16"), moe.MOE_BF16, rm, T, k, H, dxf, moe.MOE_F32)
    torch.cuda.synchronize()
    assert np.array_equal(host(dxf), pm.unpermute_sum(rows, row_map))


@pytest.mark.parametrize("fmt,R,K", [("mxfp8", 96, 160), ("mxfp8", 512, 384), ("mxfp4", 256, 96)])
def test_quantize_axis1_transposed(gpu_lib, fmt, R, K):
    log(f"axis-1 quantize {fmt} R={R} K={K}")
    g = np.random.default_rng(R + K)
    v = _bf16(g.standard_normal((R, K)) * np.exp2(g.integers(-6, 6, (R, 1))))
    v[:32, 5] = 0.0                       # an all-zero block
    codes, scales = moe.quantize_mx_t(dev(v, "bf16"), fmt)
    torch.cuda.synchronize()
    ec, es = omx.quantize(v, omx.fmt_of(fmt), axis=0)
    ec, es = ec.T, es.T                   # K-major
    if fmt == "mxfp4":
        ec = omx.pack_fp4(ec)
    assert np.array_equal(host(codes), ec)
    assert np.array_equal(host(scales), es)


def _segments_expected(vals, src, offsets, E, fmt, pad=128):
    """Oracle side of the segment-transposed quantization: per expert the
    segment's rows (zero where src < 0) padded with zero rows to a multiple
    of `pad`, MX-quantized along the rows; returns K-major codes, scales and
    the segment starts."""
    C = vals.shape[1]
    cols, scs, kofs = [], [], [0]
    for e in range(E):
        seg = vals[offsets[e]:offsets[e + 1]].copy()
        seg[src[offsets[e]:offsets[e + 1]] < 0] = 0
        n = (len(seg) + pad - 1) // pad * pad
        seg = np.concatenate([seg, np.zeros((n - len(seg), C), np.float32)])
        kofs.append(kofs[-1] + n)
        if n:
            c, s = omx.quantize(seg, omx.fmt_of(fmt), axis=0)
            cols.append(c.T)
            scs.append(s.T)
    return np.concatenate(cols, axis=1), np.concatenate(scs, axis=1), np.array(kofs)


@pytest.mark.parametrize("mode,in_fmt,scaled", [(0, "bf16", False), (0, "fp32", False),
                                                (1, "bf16", False), (1, "bf16", True),
                                                (2, "fp32", False)])
def test_quantize_segments(gpu_lib, mode, in_fmt, scaled):
    T, E, k, C = 173, 12, 3, 320
    log(f"segment quantize mode {mode} {in_fmt} scaled={scaled} T={T} E={E} C={C}")
    idx, counts, offsets, row_map, src = _maps(T, E, k, 32, 7)
    bound = len(src)
    g = np.random.default_rng(8 + mode)
    rnd = (lambda a: _bf16(a)) if in_fmt == "bf16" else (lambda a: np.asarray(a, np.float32))
    if mode == 0:
        inp = rnd(g.standard_normal((bound, C)))
        vals = inp
    elif mode == 1:
        inp = rnd(g.standard_normal((T, C)))
        vals = pm.permute_rows(inp, src)
    else:
        inp = rnd(g.standard_normal((bound, 2 * C)) * 2)
        from oracle import mlp as omlp
        vals = omlp.swiglu(inp, C)
    scale = None
    if scaled:
        rs = g.uniform(0.05, 1.0, bound).astype(np.float32)
        vals = (vals * rs[:, None]).astype(np.float32)
        scale = dev(rs)
    ks = moe.moe_segments_kstride(bound, E)
    codes = torch.zeros((C, ks), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((C, ks // 32), dtype=torch.uint8, device="cuda")
    kofs = torch.empty((E + 1,), **I32)
    moe.moe_quantize_mx_segments(dev(inp, in_fmt), moe.FMT[in_fmt], mode,
                                 torch.from_numpy(src.astype(np.int32)).cuda(),
                                 torch.from_numpy(offsets.astype(np.int32)).cuda(), scale, E, bound, C,
                                 ks, moe.MOE_MXFP8_E4M3, codes, scales, kofs)
    torch.cuda.synchronize()
    ec, es, ekofs = _segments_expected(vals, src, offsets, E, "mxfp8")
    assert np.array_equal(host(kofs), ekofs)
    n = ekofs[-1]
    gc, gs = _stage_major(host(codes), host(scales), C, ks, n)
    if mode < 2:
        assert np.array_equal(gc, ec) and np.array_equal(gs, es)
    else:
        # silu in fp32 on the device vs the oracle's: codes may differ at a
        # rounding boundary, never by more than one grid step
        assert (gs == es).mean() > 0.999
        a = omx.dequantize(gc, gs, "e4m3", axis=1)
        b = omx.dequantize(ec, es, "e4m3", axis=1)
        assert rel_l2(a, b) < 1e-3


def _stage_major(codes, scales, C, ks, n):
    """The segment quantizer's stage-major output ([ks/128][C][128] codes,
    [ks/128][C][4] scales) as K-major [C, n] codes and [C, n/32] scales."""
    c = codes.reshape(-1)[: ks * C].reshape(ks // 128, C, 128)[: n // 128]
    s = scales.reshape(-1)[: ks * C // 32].reshape(ks // 128, C, 4)[: n // 128]
    return (c.transpose(1, 0, 2).reshape(C, n), s.transpose(1, 0, 2).reshape(C, n // 32))


@pytest.mark.parametrize("M,N,T", [(256, 384, 400), (384, 256, 400), (256, 384, 2400),
                                   (1024, 2048, 400)])
def test_wgrad_ragged_segments(gpu_lib, M, N, T):
    # T = 2400 gives expert 0 more than 1024 rows: a segment longer than 8
    # stages, whose tiles are split across the XCDs instead of staying whole.
    # M = 1024, N = 2048: 128 tiles per expert, more than the 64 workgroups
    # of an XCD, so a workgroup runs consecutive tiles on the same dW rows
    # (the A block stays in LDS between them)
    E, k = 16, 4
    log(f"grouped wgrad M={M} N={N} T={T} E={E}")
    idx, counts, offsets, row_map, src = _maps(T, E, k, 32, 9)
    assert counts[0] > 256 and (counts[-3:] == 0).all()
    if T > 1000:
        assert counts[0] > 1024
    bound = len(src)
    g = np.random.default_rng(10)
    A = _bf16(g.standard_normal((bound, M)))
    B = _bf16(g.standard_normal((bound, N)))
    ks = moe.moe_segments_kstride(bound, E)
    src_d = torch.from_numpy(src.astype(np.int32)).cuda()
    off_d = torch.from_numpy(offsets.astype(np.int32)).cuda()
    kofs = torch.empty((E + 1,), **I32)
    bufs = []
    for vals, C in ((A, M), (B, N)):
        c = torch.empty((C, ks), dtype=torch.uint8, device="cuda")
        s = torch.empty((C, ks // 32), dtype=torch.uint8, device="cuda")
        moe.moe_quantize_mx_segments(dev(vals, "bf16"), moe.MOE_BF16, 0, src_d, off_d, None, E, bound,
                                     C, ks, moe.MOE_MXFP8_E4M3, c, s, kofs)
        bufs += [c, s]
    dw = torch.full((E, M, N), 5.0, dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_wgrad(bufs[0], bufs[1], bufs[2], bufs[3], moe.MOE_MXFP8_E4M3, kofs, E, M, N, ks, dw)
    torch.cuda.synchronize()
    got = host(dw)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        live = src[lo:hi] >= 0
        a = np.where(live[:, None], A[lo:hi], 0)
        b = np.where(live[:, None], B[lo:hi], 0)
        if hi == lo:
            assert (got[e] == 0).all(), f"expert {e} has no rows: gradient must be exactly zero"
            continue
        ref = (omx.fake_quant(obw._pad_rows(a, 32), "e4m3", axis=0).T
               @ omx.fake_quant(obw._pad_rows(b, 32), "e4m3", axis=0))
        assert rel_l2(got[e], ref) < TOL, e


def _gpu_backward(cfg, x_d, wr_d, b_d, w1, w2, dout_d, staged=False):
    """Forward, then the backward: one moe_grouped_mlp_bwd call, or (staged)
    one C call per step, keeping the intermediate buffers."""
    ew = moe.ExpertWeights.from_dense(w1, w2, cfg.fmt, transposed=True)
    fw = moe.MoEForward.for_config(cfg, save_act=True, keep_logits=True)
    fw(x_d, wr_d, b_d, ew)
    bw = moe.MoEBackward(fw)
    if staged:
        bw.staged(dout_d, x_d, ew)
    else:
        bw(dout_d, x_d, ew)
    torch.cuda.synchronize()
    return fw, bw, ew


@pytest.mark.parametrize("name", ["mini_skew_mxfp8", "mini_ep8_mxfp8"])
def test_backward_reduced(gpu_lib, name):
    """Every element of dx, dW1 and dW2 against the oracle: the skewed layer
    (empty experts, experts of one 32-row block and of many) and the
    expert-parallel share (8 experts of 300 rows each, segments padded to
    320)."""
    cfg = configs.get(name)
    log(f"backward end to end {cfg.name}")
    h, d = device_inputs(cfg)
    # (the one-call moe_grouped_mlp_bwd)
    fw, bw, ew = _gpu_backward(cfg, d["x"], d["w_router"], d["bias"], d["w1"], d["w2"], d["dout"])
    olog = rt.router_logits(h["x"], h["w_router"])
    oidx, ow, _, _ = rt.route(olog, h["bias"], cfg.n_group, cfg.topk_group, cfg.k, cfg.routed_scale)
    assert np.array_equal(host(fw.topk_idx), oidx)
    ref = obw.moe_backward(h["x"], h["dout"], oidx, ow, lambda e: h["w1"][e], lambda e: h["w2"][e],
                           E=cfg.E, fmt=cfg.fmt)
    dx = host(bw.dx)
    err = rel_l2(dx, ref["dx"])
    log(f"  dx rel L2 {err:.2e}")
    assert err < TOL
    counts = np.bincount(oidx.ravel(), minlength=cfg.E)
    if cfg.bias_kind == "zipf":
        assert (counts == 0).sum() >= 1, "the skewed routing leaves some experts without rows"
    else:
        assert (counts == cfg.T).all(), "top-8 of 8 experts: every expert gets every token"
    dw1, dw2 = host(bw.dw1), host(bw.dw2)
    for e in range(cfg.E):
        if counts[e] == 0:
            assert (dw1[e] == 0).all() and (dw2[e] == 0).all()
    e1 = rel_l2(dw1, np.stack([ref["dw1"][e] for e in range(cfg.E)]))
    e2 = rel_l2(dw2, np.stack([ref["dw2"][e] for e in range(cfg.E)]))
    log(f"  dW1 rel L2 {e1:.2e}, dW2 rel L2 {e2:.2e}")
    assert e1 < TOL and e2 < TOL
    # per-expert bar for every expert with rows
    for e in np.nonzero(counts)[0]:
        assert rel_l2(dw1[e], ref["dw1"][e]) < TOL and rel_l2(dw2[e], ref["dw2"][e]) < TOL, e
    # the same backward one C call per step gives the same bits
    first = [t.clone() for t in (bw.dx, bw.dw1, bw.dw2)]
    bw.staged(d["dout"], d["x"], ew)
    torch.cuda.synchronize()
    for name, a, b in zip(["dx", "dW1", "dW2"], first, (bw.dx, bw.dw1, bw.dw2)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name


def test_backward_empty_batch(gpu_lib):
    """T = 0: moe_grouped_mlp_bwd writes exact zeros to every weight
    gradient and nothing else."""
    cfg = dataclasses.replace(configs.get("mini_skew_mxfp8"), T=0)
    log("backward with T = 0")
    h, d = device_inputs(dataclasses.replace(cfg, T=1))
    ew = moe.ExpertWeights.from_dense(d["w1"], d["w2"], cfg.fmt, transposed=True)
    fw = moe.MoEForward.for_config(cfg, save_act=True)
    fw.route(d["x"][:0], d["w_router"], d["bias"])
    fw.permute()                  # empty segments; every row is padding
    fw.act_save.zero_()
    bw = moe.MoEBackward(fw)
    bw.dw1.fill_(3.0)
    bw.dw2.fill_(3.0)
    bw(d["dout"][:0], d["x"][:0], ew)
    torch.cuda.synchronize()
    assert not bw.dw1.any().item() and not bw.dw2.any().item()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["dsv4_skew_mxfp8_t8192", "dsv3_ep8_mxfp8_t4096"])
def test_backward_full_size_sampled(gpu_lib, name):
    cfg = configs.get(name)
    log(f"full-size backward {cfg.name}: generating weights on the device")
    x, wr, b = gen.host_x(cfg), gen.host_router(cfg), gen.host_bias(cfg)
    dout = gen.host_dout(cfg)
    wts = gen.device_expert_weights(cfg, "cuda")
    x_d = dev(x, "bf16")
    fw, bw, ew = _gpu_backward(cfg, x_d, dev(wr, "bf16"), dev(b), wts["w1"], wts["w2"],
                               dev(dout, "bf16"), staged=True)
    log("  forward + backward done; oracle routing of all tokens")
    olog = rt.router_logits(x, wr)
    oidx, ow, os_, osel = rt.route(olog, b, cfg.n_group, cfg.topk_group, cfg.k, cfg.routed_scale)
    idx = host(fw.topk_idx)
    nbad, unc, bad_tok = certified_tie_mismatches(osel, idx, oidx, cfg.n_group, cfg.topk_group,
                                                  margin=tie_margin(host(fw.logits), olog))
    log(f"  routing: {nbad} certified near-tie tokens, {unc} uncertified")
    assert unc == 0 and nbad <= max_tie_tokens(cfg.T, cfg.bias_kind)
    # the oracle follows the GPU's expert lists (identical but for certified
    # ties), with its own normalized scores as combine weights
    w_or = rt.combine_weights(os_, idx, cfg.routed_scale)
    counts = np.bincount(idx.ravel(), minlength=cfg.E)
    dw1_d, dw2_d = bw.dw1, bw.dw2
    zero = [e for e in range(cfg.E) if counts[e] == 0]
    assert len(zero) >= 1 or cfg.bias_kind != "zipf"
    for e in zero:
        assert not dw1_d[e].any().item() and not dw2_d[e].any().item(), e
    # skewed batch: the busiest expert (all its rows: several row tiles in the
    # data-gradient GEMMs, weight-gradient tiles split across the XCDs), a
    # mid-size one and a light one (one or two 32-row blocks); expert-parallel
    # share: two of its 8 experts of 4096 rows. Oracle backward of all their
    # rows.
    nz = np.nonzero(counts)[0]
    if cfg.bias_kind == "zipf":
        heavy = int(np.argmax(counts))
        mid = int(nz[np.argsort(counts[nz], kind="stable")[len(nz) // 2]])
        light = int([e for e in nz if 20 <= counts[e] <= 60][0])
        check = [heavy, mid, light]
    else:
        check = [0, cfg.E - 3]
    row_map = host(fw.row_map)
    from oracle import mlp as omlp
    lock = __import__("threading").Lock()

    def w_host(name_, e):
        with lock:
            u = wts[name_][e].view(torch.int16).cpu().numpy()
        return gen.bf16_bits_to_f32(u.view(np.uint16))

    def one(e):
        tj = np.argwhere(idx == e)
        t, j = tj[:, 0], tj[:, 1]
        w1, w2 = w_host("w1", e), w_host("w2", e)
        dy = (w_or[t, j][:, None].astype(np.float32) * dout[t]).astype(np.float32)
        a_ref = omlp.operand(x[t], cfg.fmt) @ omlp.operand(w1, cfg.fmt).T
        return (e, t, j, a_ref) + obw.expert_backward(x[t], dy, w1, w2, cfg.fmt)

    log(f"  oracle backward of experts {check} (rows {counts[check].tolist()}), concurrently")
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=len(check)) as ex:
        results = list(ex.map(one, check))
    worst = 0.0
    for e, t, j, a_ref, dx_e, dw1_e, dw2_e in results:
        rows = torch.from_numpy(row_map[t, j]).cuda()
        # the forward's saved fc1 output of these rows (isolates fc1)
        e_a = rel_l2(host(fw.act_save[rows]), a_ref)
        e_dx = rel_l2(host(bw.dx_perm[rows]), dx_e)
        e_w1 = rel_l2(host(dw1_d[e]), dw1_e)
        e_w2 = rel_l2(host(dw2_d[e]), dw2_e)
        log(f"  expert {e} ({len(t)} rows): saved fc1 output {e_a:.2e}, dX rows {e_dx:.2e}, "
            f"dW1 {e_w1:.2e}, dW2 {e_w2:.2e}")
        assert e_a < 1e-4
        assert e_dx < TOL and e_w1 < TOL and e_w2 < TOL
        worst = max(worst, e_w1, e_w2)
    log(f"  worst per-expert dW error {worst:.2e}")
    # un-permute property on sampled tokens: dx[t] = bf16(sum_j dX_rows[row_map[t, j]])
    g = np.random.default_rng(3)
    toks = g.choice(cfg.T, 64, replace=False)
    rm = host(fw.row_map)[toks]
    rows_h = host(bw.dx_perm[torch.from_numpy(rm.ravel()).cuda()]).reshape(len(toks), cfg.k, cfg.H)
    acc = np.zeros((len(toks), cfg.H), np.float32)
    for jj in range(cfg.k):
        acc = (acc + rows_h[:, jj]).astype(np.float32)
    assert np.array_equal(host(bw.dx[torch.from_numpy(toks).cuda()]), _bf16(acc))
    assert np.isfinite(host(bw.dx)).all()
    # a second, staged backward of the same inputs gives the same bits (row
    # fingerprints of the weight gradients, whole dA and dX rows), and the
    # one-call backward (moe_grouped_mlp_bwd) the same dx and weight
    # gradients as the staged calls
    del wts
    fp = lambda t: t.view(torch.int16).reshape(-1, t.shape[-1]).sum(dim=1, dtype=torch.int64)
    used = int(fw.offsets[-1].item())          # rows past the last segment are never written
    first = (bw.da_f32[:used].clone(), bw.dx_perm[:used].clone(), fp(bw.dw1), fp(bw.dw2),
             bw.dx.clone())
    for t_ in (bw.dw1, bw.dw2, bw.dx_perm, bw.da_f32, bw.dx):
        t_.zero_()
    bw.staged(dev(dout, "bf16"), x_d, ew)
    torch.cuda.synchronize()
    again = (bw.da_f32[:used], bw.dx_perm[:used], fp(bw.dw1), fp(bw.dw2), bw.dx)
    bits = lambda t: t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)
    same = lambda a, b_: torch.equal(bits(a) if a.dtype != torch.int64 else a,
                                     bits(b_) if b_.dtype != torch.int64 else b_)
    for name, a, b_ in zip(["dA fp32", "dX rows", "dW1 rows", "dW2 rows", "dx"], first, again):
        assert same(a, b_), name
    for t_ in (bw.dw1, bw.dw2, bw.dx):
        t_.zero_()
    bw(dev(dout, "bf16"), x_d, ew)
    torch.cuda.synchronize()
    for name, a, b_ in zip(["dW1 rows", "dW2 rows", "dx"], first[2:], (fp(bw.dw1), fp(bw.dw2), bw.dx)):
        assert same(a, b_), f"one-call backward: {name}"
