"""Helpers shared by the GPU parity tests: host<->device conversion of the
seeded inputs and the oracle runs they are compared against."""
from __future__ import annotations

import sys

import numpy as np
import torch

from moe_synth import gen


def log(msg: str):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, dtype: str = "fp32", device="cuda") -> torch.Tensor:
    """fp32 values (exactly representable in `dtype`) -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to(device)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    d = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (d if d > 0 else 1.0))


def ulp_diff_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


def device_inputs(cfg, seed=0, device="cuda"):
    """Inputs of a small or reduced config, drawn on the host and uploaded;
    returns (host dict, device dict)."""
    h = gen.host_inputs(cfg, seed)
    dt = cfg.act_dtype
    d = {"x": dev(h["x"], dt, device), "w_router": dev(h["w_router"], dt, device),
         "bias": dev(h["bias"], "fp32", device),
         "w1": dev(h["w1"], dt, device), "w2": dev(h["w2"], dt, device)}
    if cfg.n_shared:
        d["w1s"] = dev(h["w1s"], dt, device)
        d["w2s"] = dev(h["w2s"], dt, device)
    if cfg.backward:
        d["dout"] = dev(h["dout"], dt, device)
    return h, d


def tie_margin(logits_gpu: np.ndarray, logits_orc: np.ndarray) -> float:
    """How far one selection score (sel = fp32(sigmoid(logit)) + b) can move
    between the two sides, from the largest measured logit difference d:
    the sigmoid's slope is at most 1/4, and each side rounds s and s + b to
    fp32 once (at most 2^-23 apiece for values below 2). Two candidates can
    trade places only when the oracle's scores lie within twice this of each
    other."""
    d = float(np.max(np.abs(np.asarray(logits_gpu, np.float64) - np.asarray(logits_orc, np.float64)),
                     initial=0.0))
    return 0.25 * d + 2.0 ** -22


def max_tie_tokens(T: int, bias_kind: str = "uniform") -> int:
    """Tokens whose routing may differ under certified near ties: 1e-4 of
    the batch (at least one) with a random bias. A bias calibrated on the
    batch itself to equalize expert loads (the Zipf workloads) parks many
    tokens right at the k-th selection boundary, so there 5e-4 (measured on
    the 8192-token skewed batch: 3 tokens, all within the measured margin)."""
    frac = 5e-4 if bias_kind == "zipf" else 1e-4
    return max(1, int(np.ceil(T * frac)))


def certified_tie_mismatches(oracle_sel: np.ndarray, idx_gpu: np.ndarray, idx_orc: np.ndarray,
                             n_group: int = 1, topk_group: int = 1, *, margin: float):
    """Tokens whose GPU and oracle expert lists differ. The router GEMM sums
    H products in fp32 on the GPU and in fp64 in the oracle, so selection
    scores may differ by up to `margin` (tie_margin of the measured logits)
    per side; a mismatch is accepted ("certified") only when the oracle's own
    scores show a near tie that explains it: every swapped expert lies within
    2 * margin of the oracle's k-th selected score (or, for a reordering of
    the same experts, each swapped pair within 2 * margin of each other), or
    (grouped routing) the last kept and the first dropped group scores, each
    a sum of two selection scores, lie within 4 * margin + 2^-22.
    margin = 0 accepts no mismatch. Returns (n_mismatch, n_uncertified,
    mismatched token indices)."""
    from oracle import routing as rt
    bad = np.nonzero((idx_gpu != idx_orc).any(axis=1))[0]
    unc = 0
    m_e = 2.0 * margin
    m_g = 4.0 * margin + 2.0 ** -22
    for t in bad:
        if margin <= 0:
            unc += 1
            continue
        sel = oracle_sel[t].astype(np.float64)
        kth = sel[idx_orc[t, -1]]
        swapped = set(int(e) for e in idx_gpu[t]) ^ set(int(e) for e in idx_orc[t])
        ok = all(abs(sel[e] - kth) <= m_e for e in swapped)
        if set(idx_gpu[t]) == set(idx_orc[t]):
            ok = all(abs(sel[a] - sel[b]) <= m_e for a, b in zip(idx_gpu[t], idx_orc[t]))
        if not ok and n_group > 1:
            gs = np.sort(rt.group_scores(oracle_sel[t:t + 1].astype(np.float32), n_group)[0])[::-1]
            ok = abs(float(gs[topk_group - 1]) - float(gs[topk_group])) <= m_g
        unc += 0 if ok else 1
    return len(bad), unc, bad


def oracle_workers() -> int:
    """Threads for the oracle's per-expert loop at full size (the host
    cores this process may use, at most 16)."""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))
