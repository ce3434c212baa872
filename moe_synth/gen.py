"""Seeded synthetic inputs shared by the oracle and the HIP path.

This module draws random tensors and converts storage types; it holds none
of the layer's arithmetic (no routing, permutation, quantization or MLP).

Every tensor gets its own stream, keyed by (seed, config family, tensor id,
expert), so configs of one family see identical draws (the decode config
reuses the router, bias, weights and first rows of hidden states of its
4096-token parent).

Two back ends draw the same *kinds* of tensors:
  * host (numpy): everything for the small and reduced configs, and the
    hidden states, router weight, bias and upstream gradient of every config;
  * device (torch on a GPU): the expert weights of the full-size configs,
    drawn per expert with a seeded torch generator. Tests that need some of
    those weights on the host copy them back from the device tensor.
"""
from __future__ import annotations

import os
import zlib

import numpy as np

from .configs import MoEConfig, ALL

TENSOR_IDS = {"x": 1, "w_router": 2, "bias": 3, "w1": 4, "w2": 5, "w1s": 6,
              "w2s": 7, "dout": 8, "zipf_perm": 9}

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "tests", "golden")


def _family_id(family: str) -> int:
    return zlib.crc32(family.encode()) & 0x7FFFFFFF


def rng(cfg: MoEConfig, tensor: str, idx: int = 0, seed: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([seed, _family_id(cfg.family), TENSOR_IDS[tensor], idx])
    return np.random.default_rng(ss)


def torch_seed(cfg: MoEConfig, tensor: str, idx: int = 0, seed: int = 0) -> int:
    ss = np.random.SeedSequence([seed, _family_id(cfg.family), TENSOR_IDS[tensor], idx, 7])
    return int(ss.generate_state(1, np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)


# -- storage-type conversion (round to nearest even, as a tensor generator
#    would do when it emits bf16 samples) ------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 values exactly representable in the storage type `dtype`."""
    a = np.asarray(a, dtype=np.float32)
    if dtype == "fp32":
        return a
    return bf16_bits_to_f32(f32_to_bf16_bits(a))


def _normal(g: np.random.Generator, shape, std: float) -> np.ndarray:
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


# -- host draws ---------------------------------------------------------------
def host_x(cfg: MoEConfig, seed: int = 0) -> np.ndarray:
    """Hidden states [T, H] as fp32 values of the storage type."""
    if cfg.x_rows_from:
        parent = ALL[cfg.x_rows_from]
        return host_x(parent, seed)[: cfg.T].copy()
    x = _normal(rng(cfg, "x", 0, seed), (cfg.T, cfg.H), cfg.x_std)
    return round_to_storage(x, cfg.act_dtype)


def host_router(cfg: MoEConfig, seed: int = 0) -> np.ndarray:
    """Router weight [E, H]; bf16 values except in the fp32 layer."""
    w = _normal(rng(cfg, "w_router", 0, seed), (cfg.E, cfg.H), cfg.router_std)
    return round_to_storage(w, cfg.act_dtype)


def host_bias(cfg: MoEConfig, seed: int = 0) -> np.ndarray:
    """Per-expert selection bias [E] fp32."""
    if cfg.bias_kind == "uniform":
        g = rng(cfg, "bias", 0, seed)
        return g.uniform(-cfg.bias_range, cfg.bias_range, cfg.E).astype(np.float32)
    if cfg.bias_kind == "zipf":
        return load_zipf_bias(cfg, seed)
    raise ValueError(cfg.bias_kind)


def zipf_rank_permutation(cfg: MoEConfig, seed: int = 0) -> np.ndarray:
    """perm[r] = the expert that gets popularity rank r (0 = most popular)."""
    return rng(cfg, "zipf_perm", 0, seed).permutation(cfg.E).astype(np.int64)


def zipf_bias_path(cfg: MoEConfig, seed: int = 0) -> str:
    return os.path.join(GOLDEN_DIR, f"zipf_bias_{cfg.name}_seed{seed}.txt")


def load_zipf_bias(cfg: MoEConfig, seed: int = 0) -> np.ndarray:
    """The calibrated Zipf bias, stored as exact fp32 bit patterns (hex).
    It is written by the oracle package's calibration script."""
    path = zipf_bias_path(cfg, seed)
    vals = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            vals.append(int(line, 16))
    b = np.array(vals, dtype=np.uint32).view(np.float32)
    if b.shape != (cfg.E,):
        raise ValueError(f"{path}: expected {cfg.E} values, got {b.shape}")
    return b


def host_expert_w1(cfg: MoEConfig, e: int, seed: int = 0) -> np.ndarray:
    """fc1 weight of expert e, [2F, H]: rows [0, F) gate, rows [F, 2F) up."""
    w = _normal(rng(cfg, "w1", e, seed), (2 * cfg.F, cfg.H), cfg.w1_std)
    return round_to_storage(w, cfg.act_dtype)


def host_expert_w2(cfg: MoEConfig, e: int, seed: int = 0) -> np.ndarray:
    """fc2 weight of expert e, [H, F]."""
    w = _normal(rng(cfg, "w2", e, seed), (cfg.H, cfg.F), cfg.w2_std)
    return round_to_storage(w, cfg.act_dtype)


def host_shared_w1(cfg: MoEConfig, seed: int = 0) -> np.ndarray:
    w = _normal(rng(cfg, "w1s", 0, seed), (2 * cfg.F_shared, cfg.H), cfg.w1_std)
    return round_to_storage(w, cfg.act_dtype)


def host_shared_w2(cfg: MoEConfig, seed: int = 0) -> np.ndarray:
    w = _normal(rng(cfg, "w2s", 0, seed), (cfg.H, cfg.F_shared), cfg.w2s_std)
    return round_to_storage(w, cfg.act_dtype)


def host_dout(cfg: MoEConfig, seed: int = 0) -> np.ndarray:
    """Upstream gradient [T, H], N(0, 1) in the storage type."""
    d = _normal(rng(cfg, "dout", 0, seed), (cfg.T, cfg.H), 1.0)
    return round_to_storage(d, cfg.act_dtype)


def host_inputs(cfg: MoEConfig, seed: int = 0, with_weights: bool = True) -> dict:
    """All inputs of a small or reduced config on the host, as fp32 arrays
    holding values of the storage type."""
    d = {"x": host_x(cfg, seed), "w_router": host_router(cfg, seed),
         "bias": host_bias(cfg, seed)}
    if with_weights:
        d["w1"] = np.stack([host_expert_w1(cfg, e, seed) for e in range(cfg.E)])
        d["w2"] = np.stack([host_expert_w2(cfg, e, seed) for e in range(cfg.E)])
        if cfg.n_shared:
            d["w1s"] = host_shared_w1(cfg, seed)
            d["w2s"] = host_shared_w2(cfg, seed)
    if cfg.backward:
        d["dout"] = host_dout(cfg, seed)
    return d


# -- device draws (full-size expert weights) ----------------------------------
def device_expert_weights(cfg: MoEConfig, device, seed: int = 0, which=("w1", "w2")):
    """Expert weights drawn on the GPU with seeded torch generators, one
    stream per (tensor, expert). Returns {name: tensor [E, rows, cols]} in the
    storage type (bf16 except in the fp32 layer)."""
    import torch
    tdt = torch.float32 if cfg.act_dtype == "fp32" else torch.bfloat16
    shapes = {"w1": ((2 * cfg.F, cfg.H), cfg.w1_std), "w2": ((cfg.H, cfg.F), cfg.w2_std)}
    out = {}
    for name in which:
        (r, c), std = shapes[name]
        t = torch.empty((cfg.E, r, c), dtype=tdt, device=device)
        g = torch.Generator(device=device)
        for e in range(cfg.E):
            g.manual_seed(torch_seed(cfg, name, e, seed))
            tmp = torch.randn((r, c), generator=g, device=device, dtype=torch.float32)
            t[e].copy_(tmp.mul_(std))
        out[name] = t
    return out


def device_shared_weights(cfg: MoEConfig, device, seed: int = 0):
    import torch
    tdt = torch.float32 if cfg.act_dtype == "fp32" else torch.bfloat16
    out = {}
    for name, (r, c), std in (("w1s", (2 * cfg.F_shared, cfg.H), cfg.w1_std),
                              ("w2s", (cfg.H, cfg.F_shared), cfg.w2s_std)):
        g = torch.Generator(device=device)
        g.manual_seed(torch_seed(cfg, name, 0, seed))
        tmp = torch.randn((r, c), generator=g, device=device, dtype=torch.float32)
        out[name] = tmp.mul_(std).to(tdt)
    return out
