"""The seeded generators and the stored Zipf bias of the skewed workloads.

Generators: draws are deterministic per (seed, family, tensor, expert), the
bf16 storage rounding equals torch's round-to-nearest-even conversion, and
the decode config's inputs are the first rows of its parent's.
Zipf bias: re-routing the batch with the oracle reproduces the skew the
workload asks for (busiest expert far above the mean, some experts empty).
"""
import numpy as np
import pytest
import torch

from moe_synth import configs, gen
from oracle import routing as rt


def test_bf16_rounding_matches_torch():
    v = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 3
    v[:4] = [1.00390625, 1.01171875, -1.00390625, 65504.0]   # exact halfway cases
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gen.f32_to_bf16_bits(v), ref)


def test_determinism_and_family_reuse():
    a = gen.host_x(configs.get("mini_bf16"))
    b = gen.host_x(configs.get("mini_bf16"))
    assert np.array_equal(a, b)
    dec = gen.host_x(configs.get("mini_mxfp8_decode"))
    assert np.array_equal(dec, a[:dec.shape[0]])
    assert np.array_equal(gen.host_expert_w1(configs.get("mini_mxfp8_decode"), 3),
                          gen.host_expert_w1(configs.get("mini_bf16"), 3))
    assert not np.array_equal(gen.host_expert_w1(configs.get("mini_bf16"), 3),
                              gen.host_expert_w1(configs.get("mini_bf16"), 4))


def test_storage_types():
    x = gen.host_x(configs.get("mini_bf16"))
    assert (x.view(np.uint32) & 0xFFFF == 0).all()
    x32 = gen.host_x(configs.get("tiny_fp32"))
    assert (x32.view(np.uint32) & 0xFFFF != 0).any()


@pytest.mark.parametrize("name,min_ratio", [("mini_skew_mxfp8", 4.0), ("dsv4_skew_mxfp8_t8192", 10.0)])
def test_zipf_bias_gives_skew(name, min_ratio):
    cfg = configs.get(name)
    x = gen.host_x(cfg)
    wr = gen.host_router(cfg)
    b = gen.host_bias(cfg)
    idx, _, _, _ = rt.route(rt.router_logits(x, wr), b, 1, 1, cfg.k, cfg.routed_scale)
    counts = np.bincount(idx.ravel(), minlength=cfg.E)
    mean = cfg.T * cfg.k / cfg.E
    assert counts.max() >= min_ratio * mean
    assert (counts == 0).sum() >= cfg.n_zero_experts
