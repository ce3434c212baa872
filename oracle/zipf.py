"""Calibration of the selection bias that makes expert popularity Zipf-skewed.

TEST INFRASTRUCTURE ONLY (it writes a stored input under tests/golden/ and
calls nothing but the oracle and the seeded generators).

The skewed workload asks for expert popularity following Zipf(s) so that
some experts get more than ten times the mean rows and some get none. The
bias is the aux-loss-free selection bias of [TE-DSV3] (Description,
DeepSeekV3MoE item), here used as the knob. Steps:
  1. target rows c_r proportional to r^-s over popularity ranks r = 1..E
     (rank -> expert by a seeded permutation), scaled to sum T*k and capped
     at T rows per expert by water-filling;
  2. starting from b = 0, a fixed number of sign updates
     b_e += gamma_i * sign(c_e - load_e(b)) with a geometrically decaying
     step gamma_i, where load_e is the oracle's routing of this very batch;
  3. the n_zero least popular experts get b = -(max|b| + 2), which puts
     them below every other expert (scores lie in (0, 1));
  4. the stored bias is accepted if the busiest expert gets at least
     `min_ratio` times the mean rows and at least one expert gets none.

Usage: python -m oracle.zipf <config name> [seed]
"""
from __future__ import annotations

import sys

import numpy as np

from . import routing as _rt


def zipf_targets(E: int, total: int, cap: int, s: float) -> np.ndarray:
    """Water-filled targets by popularity rank (rank 0 = most popular)."""
    p = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    c = np.zeros(E)
    capped = np.zeros(E, dtype=bool)
    for _ in range(E):
        rest = total - cap * capped.sum()
        c = np.where(capped, cap, rest * p / p[~capped].sum())
        over = (c > cap) & ~capped
        if not over.any():
            break
        capped |= over
    return c


def loads(s: np.ndarray, bias: np.ndarray, k: int) -> np.ndarray:
    sel = _rt.selection_scores(s, bias)
    idx = _rt.topk_desc(sel, k)
    return np.bincount(idx.ravel(), minlength=s.shape[1])


def calibrate(cfg, seed: int = 0, iters: int = 400, gamma0: float = 0.05,
              gamma1: float = 2e-4):
    from moe_synth import gen
    x = gen.host_x(cfg, seed)
    wr = gen.host_router(cfg, seed)
    s = _rt.sigmoid_scores(_rt.router_logits(x, wr))
    perm = gen.zipf_rank_permutation(cfg, seed)
    n_live = cfg.E - cfg.n_zero_experts
    target = np.zeros(cfg.E)
    target[perm[:n_live]] = zipf_targets(n_live, cfg.T * cfg.k, cfg.T, cfg.zipf_s)
    b = np.zeros(cfg.E, dtype=np.float32)
    for i in range(iters):
        g = gamma0 * (gamma1 / gamma0) ** (i / max(1, iters - 1))
        ld = loads(s, b, cfg.k)
        b = (b + np.float32(g) * np.sign(target - ld).astype(np.float32)).astype(np.float32)
    dead = perm[n_live:]
    b[dead] = -(np.abs(b).max() + np.float32(2))
    return b.astype(np.float32), target, loads(s, b, cfg.k)


def write(cfg, seed: int = 0, min_ratio: float = 10.0):
    from moe_synth import gen
    b, target, ld = calibrate(cfg, seed)
    mean = cfg.T * cfg.k / cfg.E
    ratio = ld.max() / mean
    if ratio < min_ratio or (ld == 0).sum() == 0:
        raise RuntimeError(f"calibration missed: max/mean {ratio:.1f}, zeros {(ld == 0).sum()}")
    path = gen.zipf_bias_path(cfg, seed)
    with open(path, "w") as f:
        f.write(f"# selection bias for {cfg.name} seed {seed}: fp32 bit patterns, one per expert\n")
        f.write(f"# written by: python -m oracle.zipf {cfg.name} {seed}\n")
        f.write(f"# realized rows: max {ld.max()} ({ratio:.1f}x mean {mean:.1f}), "
                f"zero-row experts {(ld == 0).sum()}\n")
        for v in b.view(np.uint32):
            f.write(f"{int(v):08x}\n")
    return path, ld


if __name__ == "__main__":
    from moe_synth import configs
    cfg = configs.get(sys.argv[1])
    seed = int(sys.argv[2]) if len(sys.argv) > 2 else 0
    ratio = 10.0 if cfg.E / cfg.k > 20 else 4.0
    path, ld = write(cfg, seed, min_ratio=ratio)
    print(path, "max rows", ld.max(), "zero experts", int((ld == 0).sum()))
