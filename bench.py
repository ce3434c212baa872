"""Throughput of the routed MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--cpu-experts M]
    python bench.py --copy-calibration MIB

The second form only runs a plain device-to-device copy of MIB MiB a few
times: under rocprofv3 --pmc it gives the FETCH_SIZE / WRITE_SIZE readings
of a known byte count, the scale for the layer kernels' readings.

A step is one whole pass of the layer over one batch of synthetic inputs
that are resident in HBM before timing starts: router GEMM + grouped top-k,
MX quantization of the hidden states (MX workloads), permute maps, grouped
fc1 + SwiGLU, grouped fc2, shared expert, combine; for the workload with a
backward also the whole backward (combine backward with the dY quantization,
fc2 data gradient fused with the SwiGLU backward, fc1 data gradient,
un-permute, segment quantizations and both weight-gradient GEMMs). W untimed
warm-up steps, then exactly K timed steps bracketed by device
synchronization. One JSON line is printed.

The default workload is DeepSeek-V3 dims at 4096 tokens, bf16 (hidden 7168,
expert FFN 2048, 256 experts in 8 groups, top-4 groups, top-8, routed scale
2.5, one shared expert). --workload picks another configuration of the
layer; its line carries its own name in config.workload.

Inside the timed region every stage is bracketed by HIP events on the stream
its kernels are launched on. The stage with the largest average duration is
the dominant kernel of the roofline entry: its algorithmic bytes and flops
per launch (weights of the experts that received rows read once, activation
rows read or written once, in their storage formats) decide the bound
(arithmetic intensity against the ridge of the format's MFMA peak over the
8 TB/s HBM peak) and the achieved rate. `traffic` is the HBM bytes per
launch of that kernel measured with rocprofv3 counters (profiles/
pmc_<stage>_<workload>.txt, scaled by the copy calibration), reported only
while the kernel source is the one that was measured (its SHA-256 is
recorded in that file), else null. The CPU baseline times the oracle (plain
numpy, BLAS on every usable host core) on a bounded sample of the same
batch: routing of every token, the expert MLPs of a few whole experts (all
their rows), a share of the shared expert and the whole combine, scaled to
the batch by the number of touched experts (see cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

METRIC = "MoE layer tokens/s + TFLOP/s (% MFMA peak) at DSV3 dims, 4096 tok, 1 GPU"
# the NVFP4 GEMMs run bf16 matrix instructions on exact bf16 operand values
PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0, "mxfp4": 10100.0, "fp32": 157.3, "nvfp4": 2500.0}
PEAK_HBM_GBS = 8000.0
# bytes per stored element (MX: code + one scale byte per 32 elements)
ELEM_BYTES = {"bf16": 2.0, "fp32": 4.0, "mxfp8": 1 + 1 / 32, "mxfp4": 0.5 + 1 / 32,
              "nvfp4": 0.5 + 1 / 16}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def stage_work(cfg, counts: np.ndarray, backward: bool, kpad: int = 0, fused_shared: bool = False):
    """Algorithmic (bytes, flops) per launch of each timed stage. kpad: the
    padded length of the weight-gradient contraction (the segment rows, each
    segment padded to 128), which the stage-major operands hold.
    fused_shared: the shared expert runs inside the fc1 / fc2 launches."""
    T, H, F, E, k = cfg.T, cfg.H, cfg.F, cfg.E, cfg.k
    R = T * k                                   # token-expert rows
    touched = int((counts > 0).sum())
    wb = ELEM_BYTES[cfg.fmt]
    ab = ELEM_BYTES[cfg.act_dtype]              # bf16 / fp32 activations
    qb = wb                                     # layer-format activation rows
    work = {}
    work["route"] = (T * H * ab + E * H * ab + T * k * 8, 2.0 * T * H * E)
    if cfg.fmt in ("mxfp8", "mxfp4", "nvfp4"):
        work["quantize_x"] = (T * H * ab + T * H * qb, 0.0)
    work["permute"] = (T * k * 4 * 3 + E * 8, 0.0)
    save = R * 2 * F * 4 if backward else 0
    work["fc1_swiglu"] = (touched * 2 * F * H * wb + T * H * qb + R * F * qb + save,
                          2.0 * R * H * 2 * F)
    work["fc2"] = (touched * H * F * wb + R * F * qb + R * H * ab, 2.0 * R * F * H)
    if cfg.n_shared and fused_shared:
        # x rows are read once for both; the shared h goes through HBM
        Fs = cfg.F_shared
        b1, f1 = work["fc1_swiglu"]
        work["fc1_swiglu"] = (b1 + 2 * Fs * H * wb + T * Fs * qb, f1 + 2.0 * T * H * 2 * Fs)
        b2, f2 = work["fc2"]
        work["fc2"] = (b2 + H * Fs * wb + T * Fs * qb + T * H * ab, f2 + 2.0 * T * Fs * H)
    elif cfg.n_shared:
        Fs = cfg.F_shared
        work["shared"] = (2 * Fs * H * wb + H * Fs * wb + T * H * qb + T * H * ab,
                          2.0 * T * H * 2 * Fs + 2.0 * T * Fs * H)
    work["combine"] = (R * H * ab + T * H * ab * (2 if cfg.n_shared else 1), 0.0)
    if backward:
        work["combine_bwd"] = (R * H * ab + R * H * qb, 0.0)
        work["fc2_dgrad_dswiglu"] = (touched * F * H * wb + R * H * qb + R * 2 * F * 4
                                     + R * 2 * F * (qb + 4), 2.0 * R * H * F)
        work["fc1_dgrad"] = (touched * H * 2 * F * wb + R * 2 * F * qb + R * H * 2,
                             2.0 * R * 2 * F * H)
        work["unpermute"] = (R * H * 2 + T * H * 2, 0.0)
        op2 = kpad * (H + F) * 33 // 32           # E4M3 codes + E8M0 scales
        op1 = kpad * (2 * F + H) * 33 // 32
        work["operands_dw2"] = (R * H * ab + R * 2 * F * 4 + op2, 0.0)
        work["wgrad_dw2"] = (op2 + E * H * F * 2, 2.0 * R * H * F)
        work["operands_dw1"] = (R * 2 * F * 4 + R * H * ab + op1, 0.0)
        work["wgrad_dw1"] = (op1 + E * 2 * F * H * 2, 2.0 * R * 2 * F * H)
    return work


def roofline_entry(name, nbytes, flops, ms, fmt):
    peak_f = PEAK_TFLOPS[fmt]
    ridge = peak_f * 1e12 / (PEAK_HBM_GBS * 1e9)     # flop per byte
    if flops > 0 and flops / nbytes >= ridge:
        ach = flops / (ms * 1e-3) / 1e12
        return {"kernel": name, "bound": "mfma", "achieved": round(ach, 1), "peak": peak_f,
                "unit": "TFLOP/s", "frac": round(ach / peak_f, 4), "traffic": None,
                "flops_per_launch": flops, "bytes_per_launch": nbytes,
                "avg_launch_ms": round(ms, 4)}
    ach = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": name, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None,
            "bytes_per_launch": nbytes, "flops_per_launch": flops, "avg_launch_ms": round(ms, 4)}


HERE = os.path.dirname(os.path.abspath(__file__))
# source file of each stage's dominant kernel (for the traffic record)
STAGE_SOURCE = {
    "fc1_swiglu": "expert_gemm.hip", "fc2": "expert_gemm.hip", "shared": "expert_gemm.hip",
    "fc2_dgrad_dswiglu": "expert_gemm.hip", "fc1_dgrad": "expert_gemm.hip",
    "wgrad_dw1": "wgrad.hip", "wgrad_dw2": "wgrad.hip", "route": "route.hip",
    "operands_dw1": "backward.hip", "operands_dw2": "backward.hip",
    "combine": "combine.hip", "combine_bwd": "backward.hip",
}


def source_sha(stage: str):
    name = STAGE_SOURCE.get(stage)
    if name is None:
        return None
    path = os.path.join(HERE, "mixture_experts_layer_sigmoid_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(stage: str, workload: str):
    """HBM bytes per launch from profiles/pmc_<stage>_<workload>.txt, or None
    when there is no record or the kernel source changed since."""
    path = os.path.join(HERE, "profiles", f"pmc_{stage}_{workload}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("source_sha256") != source_sha(stage):
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(mib: int):
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 3}), flush=True)


def host_info():
    """Host facts printed with every record: usable cores and CPU model."""
    cores = len(os.sched_getaffinity(0))
    model = None
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except Exception:
        pass
    return cores, model


def cpu_baseline(cfg, x, wr, b, wts, sh, dout, backward: bool, budget_experts: int | None = None):
    """Time the oracle (plain numpy) on a bounded sample of the same batch
    and scale it to the whole batch.

    The oracle's cost is a fixed part per touched expert (widening or MX
    fake-quantizing its weights) plus a part per row, so a sample of whole
    experts with all their rows scales to the batch by the count of touched
    experts: routing of every token (timed in full), the expert MLPs (and
    for the skewed workload the expert backward) of m experts picked at
    evenly spaced row-count quantiles, the shared expert on a share of the
    tokens, and the combine of every token. BLAS runs on every usable host
    core."""
    import torch
    from threadpoolctl import threadpool_limits
    from oracle import backward as obw, mlp as omlp, routing as rt
    cores, model = host_info()
    widen = lambda u: (u.astype(np.uint32) << 16).view(np.float32)
    w1_of = lambda e: widen(wts["w1"][e].view(torch.int16).cpu().numpy().view(np.uint16))
    w2_of = lambda e: widen(wts["w2"][e].view(torch.int16).cpu().numpy().view(np.uint16))
    T, k, fmt = cfg.T, cfg.k, cfg.fmt
    gx, gh = (cfg.x_global, cfg.h_global) if fmt == "nvfp4" else (None, None)
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        logits = rt.router_logits(x, wr)
        idx, w, s, sel = rt.route(logits, b, cfg.n_group, cfg.topk_group, k, cfg.routed_scale)
        t_route = time.perf_counter() - t0
        counts = np.bincount(idx.ravel(), minlength=cfg.E)
        touched = np.nonzero(counts)[0]
        if budget_experts is None:
            # bf16: the whole batch (every touched expert, the shared expert on
            # every token: a few seconds); MX / NVFP4 fake-quantization makes
            # the oracle far slower per expert, so those take a sample
            budget_experts = {"bf16": cfg.E, "mxfp8": 3, "mxfp4": 4, "nvfp4": 4}.get(fmt, 8)
            if backward:
                budget_experts = 2
        m = max(1, min(budget_experts, len(touched)))
        order = touched[np.argsort(counts[touched], kind="stable")]
        picks = order[np.linspace(0, len(order) - 1, m + 2)[1:-1].round().astype(int)] if m < len(order) \
            else order
        log(f"cpu baseline: routing {t_route:.1f} s; expert sample {picks.tolist()} "
            f"(rows {counts[picks].tolist()})")
        t_exp = 0.0
        for e in picks:
            tj = np.argwhere(idx == e)
            t_, j_ = tj[:, 0], tj[:, 1]
            w1, w2 = w1_of(int(e)), w2_of(int(e))
            t0 = time.perf_counter()
            xq = omlp.operand(x[t_], fmt, axis=-1, g=gx)
            omlp.expert_mlp(xq, omlp.operand(w1, fmt, axis=-1), omlp.operand(w2, fmt, axis=-1), fmt,
                            gh)
            if backward:
                dy = (w[t_, j_][:, None].astype(np.float32) * dout[t_]).astype(np.float32)
                obw.expert_backward(x[t_], dy, w1, w2, fmt)
            t_exp += time.perf_counter() - t0
        t_sh, n_sh = 0.0, 0
        if sh is not None:
            n_sh = T if fmt == "bf16" else min(T, 512)
            w1s, w2s = sh["w1s"].float().cpu().numpy(), sh["w2s"].float().cpu().numpy()
            t0 = time.perf_counter()
            xq = omlp.operand(x[:n_sh], fmt, axis=-1)
            omlp.expert_mlp(xq, omlp.operand(w1s, fmt), omlp.operand(w2s, fmt), fmt)
            t_sh = time.perf_counter() - t0
        y_rows = np.zeros((T * k, cfg.H), np.float32)
        t0 = time.perf_counter()
        omlp.combine(y_rows, np.arange(T * k).reshape(T, k), w)
        t_comb = time.perf_counter() - t0
        del y_rows
    total = t_route + t_exp * len(touched) / len(picks) + (t_sh * T / n_sh if n_sh else 0.0) + t_comb
    measured = t_route + t_exp + t_sh + t_comb
    what = "forward" + (" and expert backward" if backward else "")
    sample = (f"oracle {what}: routing of all {T} tokens ({t_route:.1f} s) + the expert MLPs of "
              f"{len(picks)} of the {len(touched)} touched experts with all their rows "
              f"({int(counts[picks].sum())} rows, {t_exp:.1f} s, scaled x{len(touched) / len(picks):.1f})"
              + (f" + the shared expert on {n_sh} of {T} tokens ({t_sh:.1f} s, scaled x{T / n_sh:.1f})"
                 if n_sh else "")
              + f" + the combine of all tokens ({t_comb:.1f} s); {measured:.1f} s measured, "
              f"{total:.1f} s estimated for the whole batch")
    return {"value": round(T / total, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": sample, "cpu_model": model, "seconds_estimated": round(total, 1),
            "seconds_measured": round(measured, 1)}


def run_metadata():
    """Date, source hash of the HIP library and the git commit (when the
    tree carries its .git)."""
    import datetime
    import glob
    import subprocess
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(HERE, "mixture_experts_layer_sigmoid_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    commit = None
    try:
        r = subprocess.run(["git", "-C", HERE, "rev-parse", "--short=12", "HEAD"], capture_output=True,
                           text=True, timeout=10)
        commit = r.stdout.strip() or None
    except Exception:
        pass
    return {"date_utc": datetime.datetime.utcnow().strftime("%Y-%m-%dT%H:%M:%SZ"),
            "git_commit": commit, "csrc_sha256": h.hexdigest()[:16]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3_bf16_t4096")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-experts", type=int, default=None,
                    help="experts (with all their rows) in the CPU-baseline sample")
    ap.add_argument("--copy-calibration", type=int, default=None, metavar="MIB")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the layer runs on a single MI355X with no "
              f"collectives (asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import mixture_experts_layer_sigmoid_amd as moe
    from moe_synth import configs, gen

    cfg = configs.get(args.workload)
    backward = bool(cfg.backward)
    moe.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"workload {cfg.name}: drawing inputs")
    x = gen.host_x(cfg)
    wr = gen.host_router(cfg)
    b = gen.host_bias(cfg)
    dout = gen.host_dout(cfg) if backward else None
    act = torch.float32 if cfg.act_dtype == "fp32" else torch.bfloat16
    x_d = torch.from_numpy(x).to(dev).to(act)
    wr_d = torch.from_numpy(wr).to(dev).to(act)
    b_d = torch.from_numpy(b).to(dev)
    dout_d = torch.from_numpy(dout).to(dev).to(act) if backward else None
    wts = gen.device_expert_weights(cfg, dev)
    sh = gen.device_shared_weights(cfg, dev) if cfg.n_shared else None
    # weight preparation (MX quantization, transposed copies for the
    # backward) happens once per weight update, outside the timed step
    ew = moe.ExpertWeights.from_dense(wts["w1"], wts["w2"], cfg.fmt, transposed=backward)
    sw = moe.ExpertWeights.from_dense(sh["w1s"], sh["w2s"], cfg.fmt) if sh else None
    want_cpu = not args.no_cpu_baseline
    if cfg.fmt != "bf16" and not want_cpu:
        del wts["w1"], wts["w2"]
    fw = moe.MoEForward.for_config(cfg, device=dev, save_act=backward)
    bw = moe.MoEBackward(fw) if backward else None
    if bw is not None:
        bw.stage_buffers()     # the backward is timed one C call per stage
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()

    names = ["route", "quantize_x", "permute", "fc1_swiglu", "fc2", "shared", "combine"]
    if backward:
        names += ["combine_bwd", "fc2_dgrad_dswiglu", "fc1_dgrad", "unpermute", "operands_dw2",
                  "wgrad_dw2", "operands_dw1", "wgrad_dw1"]
    if not (moe.layer.is_mx(cfg.fmt) or cfg.fmt == "nvfp4"):
        names.remove("quantize_x")
    if not cfg.n_shared or fw.fuse_shared:
        names.remove("shared")      # none, or inside fc1_swiglu / fc2
    f8 = moe.FMT["mxfp8"]

    def run_stage(name):
        if name == "route":
            fw.route(x_d, wr_d, b_d)
        elif name == "quantize_x":
            fw.quantize_x(x_d)
        elif name == "permute":
            fw.permute()
        elif name == "fc1_swiglu":
            fw.experts_fc1(x_d, ew, sw=sw)
        elif name == "fc2":
            fw.experts_fc2(ew, sw=sw)
        elif name == "shared":
            fw.shared(x_d, sw)
        elif name == "combine":
            fw.combine()
        elif name == "combine_bwd":
            moe.moe_combine_bwd(dout_d, fw.act_fmt, fw.row_map, fw.src_row, fw.topk_w, fw.T, fw.k,
                                fw.H, fw.bound, bw.dy_q, f8, bw.dy_sc, bw.row_w)
        elif name == "fc2_dgrad_dswiglu":
            moe.moe_grouped_fc2_dgrad_dswiglu(bw.dy_q, bw.dy_sc, f8, ew.w2t, ew.w2t_sc, fw.offsets,
                                              fw.E, fw.H, fw.F, fw.bound, fw.act_save, bw.da,
                                              bw.da_sc, bw.da_f32)
        elif name == "fc1_dgrad":
            moe.moe_grouped_fc1_dgrad(bw.da, bw.da_sc, f8, ew.w1t, ew.w1t_sc, fw.offsets, fw.E,
                                      fw.H, fw.F, fw.bound, bw.dx_perm)
        elif name == "unpermute":
            moe.moe_unpermute(bw.dx_perm, moe.MOE_BF16, fw.row_map, fw.T, fw.k, fw.H, bw.dx,
                              moe.MOE_BF16)
        elif name == "operands_dw2":
            bw.operands_dw2(dout_d)
        elif name == "wgrad_dw2":
            bw.gemm_dw2()
        elif name == "operands_dw1":
            bw.operands_dw1(x_d)
        elif name == "wgrad_dw1":
            bw.gemm_dw1()

    def step(evs=None):
        for i, n in enumerate(names):
            if evs is not None:
                evs[i][0].record(stream)
            run_stage(n)
            if evs is not None:
                evs[i][1].record(stream)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in names] for _ in range(args.steps)]
    log(f"timing {args.steps} steps of {len(names)} stages")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stage_ms = {n: float(np.mean([evs[s][i][0].elapsed_time(evs[s][i][1])
                                  for s in range(args.steps)])) for i, n in enumerate(names)}
    ms_per_step = elapsed * 1e3 / args.steps
    counts = fw.counts.cpu().numpy()
    kpad = int(bw.kofs[-1].item()) if backward else 0
    work = stage_work(cfg, counts, backward, kpad, fused_shared=fw.fuse_shared)

    tokens_per_s = cfg.T * args.steps / elapsed
    flops = cfg.flops_forward() + (cfg.flops_backward() if backward else 0.0)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[cfg.fmt]
    dom = max(names, key=lambda n: stage_ms[n])
    roof = roofline_entry(dom, work[dom][0], work[dom][1], stage_ms[dom], cfg.fmt)
    roof["traffic"] = measured_traffic(dom, cfg.name)
    stages = {n: {"ms": round(stage_ms[n], 4),
                  **({"gbs": round(work[n][0] / (stage_ms[n] * 1e-3) / 1e9, 1)} if n in work else {}),
                  **({"tflops": round(work[n][1] / (stage_ms[n] * 1e-3) / 1e12, 1)}
                     if n in work and work[n][1] else {})}
              for n in names}
    rec = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.fmt,
        "data": "synthetic (seeded; random-init weights of the layer's shapes)",
        "config": {"workload": cfg.name, "pass": "forward+backward" if backward else "forward",
                   "tokens": cfg.T, "hidden": cfg.H, "expert_ffn": cfg.F, "experts": cfg.E,
                   "n_group": cfg.n_group, "topk_group": cfg.topk_group, "top_k": cfg.k,
                   "routed_scale": cfg.routed_scale, "shared_experts": cfg.n_shared,
                   "experts_with_rows": int((counts > 0).sum()), "parallelism": "single GPU"},
        "tflops": round(tflops, 2),
        "mfma_peak_frac": round(tflops / peak, 4),
        "roofline": roof,
        "stages": stages,
    }
    cores, model = host_info()
    props = torch.cuda.get_device_properties(dev)
    rec["run"] = {**run_metadata(), "gpu": props.name, "gpu_cus": props.multi_processor_count,
                  "host_cores": cores, "cpu_model": model}
    if want_cpu:
        rec["cpu_baseline"] = cpu_baseline(cfg, x, wr, b, wts, sh, dout, backward, args.cpu_experts)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
