"""Throughput of the routed MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--cpu-tokens N]

A step is one whole forward pass (router GEMM + grouped top-k, permute maps,
grouped fc1 + SwiGLU, grouped fc2, shared expert, combine) over one batch of
synthetic inputs that are resident in HBM before timing starts. W untimed
warm-up steps, then exactly K timed steps bracketed by device
synchronization. One JSON line is printed.

The default workload is DeepSeek-V3 dims at 4096 tokens, bf16 (hidden 7168,
expert FFN 2048, 256 experts in 8 groups, top-4 groups, top-8, routed scale
2.5, one shared expert).
Other workloads of the same family can be chosen with --workload for study;
their lines carry their own name in config.workload.

Inside the timed region the dominant kernel (grouped fc1 + SwiGLU) is
bracketed by HIP events on the stream it is launched on; its average
duration gives the roofline entry. The CPU baseline times the oracle (plain
numpy) on the first --cpu-tokens tokens of the same batch.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "MoE layer tokens/s + TFLOP/s (% MFMA peak) at DSV3 dims, 4096 tok, 1 GPU"
PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0, "mxfp4": 10100.0, "fp32": 157.3}
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def fc1_algorithmic_bytes(cfg, counts: np.ndarray) -> float:
    """Bytes fc1 + SwiGLU must move: the fc1 weights of every expert that
    received rows (read once), the token rows (read once), and h (written
    once), in the layer's storage formats."""
    touched = int((counts > 0).sum())
    if cfg.fmt == "bf16":
        wbytes, xbytes, hbytes = 2.0, 2.0, 2.0
    elif cfg.fmt == "mxfp8":
        wbytes, xbytes, hbytes = 1 + 1 / 32, 1 + 1 / 32, 1 + 1 / 32
    elif cfg.fmt == "mxfp4":
        wbytes, xbytes, hbytes = 0.5 + 1 / 32, 0.5 + 1 / 32, 0.5 + 1 / 32
    else:
        wbytes, xbytes, hbytes = 4.0, 4.0, 4.0
    w = touched * 2 * cfg.F * cfg.H * wbytes
    x = cfg.T * cfg.H * xbytes
    h = cfg.rows * cfg.F * hbytes
    return w + x + h


def cpu_baseline(cfg, x, wr, b, wts, sh, n_tokens: int):
    """Time the oracle forward on the first n_tokens tokens (weights held on
    the host in their bf16 storage type and widened to fp32 by the oracle's
    weight accessors, as the oracle consumes them)."""
    import torch
    from oracle import mlp as omlp
    log(f"cpu baseline: copying weights to the host for {n_tokens} tokens")
    w1h = wts["w1"].view(torch.int16).cpu().numpy().view(np.uint16)
    w2h = wts["w2"].view(torch.int16).cpu().numpy().view(np.uint16)
    shared = None
    if sh is not None:
        shared = (sh["w1s"].float().cpu().numpy(), sh["w2s"].float().cpu().numpy())
    widen = lambda u: (u.astype(np.uint32) << 16).view(np.float32)
    xs = x[:n_tokens]
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    log(f"cpu baseline: oracle forward on {n_tokens} tokens, {threads} BLAS threads")
    t0 = time.perf_counter()
    omlp.moe_forward(xs, wr, b, lambda e: widen(w1h[e]), lambda e: widen(w2h[e]), E=cfg.E,
                     n_group=cfg.n_group, topk_group=cfg.topk_group, k=cfg.k,
                     routed_scale=cfg.routed_scale, fmt=cfg.fmt, shared_w=shared)
    dt = time.perf_counter() - t0
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"oracle forward (routing, {cfg.k} routed experts + shared expert, combine) "
                      f"of the first {n_tokens} tokens of the {cfg.T}-token batch; {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3_bf16_t4096")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=96)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the layer runs on a single MI355X with no "
              f"collectives (asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import mixture_experts_layer_sigmoid_amd as moe
    from moe_synth import configs, gen

    cfg = configs.get(args.workload)
    moe.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"workload {cfg.name}: drawing inputs")
    x = gen.host_x(cfg)
    wr = gen.host_router(cfg)
    b = gen.host_bias(cfg)
    act = torch.float32 if cfg.act_dtype == "fp32" else torch.bfloat16
    x_d = torch.from_numpy(x).to(dev).to(act)
    wr_d = torch.from_numpy(wr).to(dev).to(act)
    b_d = torch.from_numpy(b).to(dev)
    wts = gen.device_expert_weights(cfg, dev)
    sh = gen.device_shared_weights(cfg, dev) if cfg.n_shared else None
    ew = moe.ExpertWeights.from_dense(wts["w1"], wts["w2"], cfg.fmt)
    sw = moe.ExpertWeights.from_dense(sh["w1s"], sh["w2s"], cfg.fmt) if sh else None
    if moe.layer.is_mx(cfg.fmt):
        del wts["w1"], wts["w2"]
    fw = moe.MoEForward.for_config(cfg, device=dev)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()

    def step(ev=None):
        fw.route(x_d, wr_d, b_d)
        fw.quantize_x(x_d)
        fw.permute()
        if ev is not None:
            ev[0].record(stream)
        fw.experts_fc1(x_d, ew)
        if ev is not None:
            ev[1].record(stream)
        fw.experts_fc2(ew)
        if cfg.n_shared:
            fw.shared(x_d, sw)
        fw.combine()

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    fc1_ms = float(np.mean([a.elapsed_time(c) for a, c in evs]))
    ms_per_step = elapsed * 1e3 / args.steps
    counts = fw.counts.cpu().numpy()

    tokens_per_s = cfg.T * args.steps / elapsed
    tflops = cfg.flops_forward() / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[cfg.fmt]
    fc1_bytes = fc1_algorithmic_bytes(cfg, counts)
    achieved = fc1_bytes / (fc1_ms * 1e-3) / 1e9
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
        "config": {"workload": cfg.name, "tokens": cfg.T, "hidden": cfg.H, "expert_ffn": cfg.F,
                   "experts": cfg.E, "n_group": cfg.n_group, "topk_group": cfg.topk_group,
                   "top_k": cfg.k, "routed_scale": cfg.routed_scale,
                   "shared_experts": cfg.n_shared, "parallelism": "single GPU"},
        "tflops": round(tflops, 2),
        "mfma_peak_frac": round(tflops / peak, 4),
        "roofline": {"kernel": "grouped fc1 + SwiGLU", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "bytes_per_launch": fc1_bytes, "avg_launch_ms": round(fc1_ms, 4)},
    }
    if not args.no_cpu_baseline and cfg.fmt == "bf16":
        rec["cpu_baseline"] = cpu_baseline(cfg, x, wr, b, wts, sh, args.cpu_tokens)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
