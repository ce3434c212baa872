"""GPU parity of moe_combine against the oracle's combine: the same seeded
expert rows, maps and weights go to both sides; fp32 and bf16, with and
without a shared-expert row, and the constant-row closed form."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_sigmoid_amd as moe
from moe_synth import gen
from oracle import mlp as omlp, permute as pm
from tests.gpu_util import dev, host, log, rel_l2

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,shared,T,k,H,E", [
    ("fp32", False, 64, 4, 256, 16), ("bf16", True, 4096, 8, 7168, 256),
    ("bf16", False, 333, 6, 512, 48), ("fp32", True, 5, 1, 8, 2)])
def test_combine_parity(gpu_lib, dtype, shared, T, k, H, E):
    log(f"combine {dtype} shared={shared} T={T} k={k} H={H}")
    g = np.random.default_rng(T + H)
    idx = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _, _, row_map, src = pm.permute_maps(idx, E, 16)
    y = gen.round_to_storage(g.standard_normal((len(src), H)).astype(np.float32), dtype)
    w = g.uniform(0.05, 1.0, (T, k)).astype(np.float32)
    sh = gen.round_to_storage(g.standard_normal((T, H)).astype(np.float32), dtype) if shared else None
    f = moe.FMT[dtype]
    out = torch.empty((T, H), dtype=torch.float32 if dtype == "fp32" else torch.bfloat16, device="cuda")
    moe.moe_combine(dev(y, dtype), f, torch.from_numpy(row_map).cuda(), dev(w), None if sh is None else dev(sh, dtype),
                    T, k, H, out, f)
    torch.cuda.synchronize()
    ref = omlp.combine(y, row_map, w, sh)
    tol = 1e-6 if dtype == "fp32" else 4e-3
    assert rel_l2(host(out), ref) < tol
    # fp32 output of bf16 rows: only the accumulation order differs
    if dtype == "bf16":
        out32 = torch.empty((T, H), dtype=torch.float32, device="cuda")
        moe.moe_combine(dev(y, dtype), f, torch.from_numpy(row_map).cuda(), dev(w),
                        None if sh is None else dev(sh, dtype), T, k, H, out32, moe.MOE_F32)
        torch.cuda.synchronize()
        assert rel_l2(host(out32), ref) < 1e-6


def test_constant_rows_closed_form(gpu_lib):
    T, k, H, E = 100, 8, 64, 32
    g = np.random.default_rng(1)
    idx = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _, _, row_map, src = pm.permute_maps(idx, E, 1)
    y = np.full((len(src), H), 3.0, np.float32)
    w = np.full((T, k), np.float32(2.5 / 8), np.float32)
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    moe.moe_combine(dev(y), moe.MOE_F32, torch.from_numpy(row_map).cuda(), dev(w), None, T, k, H, out,
                    moe.MOE_F32)
    torch.cuda.synchronize()
    assert (host(out) == np.float32(7.5)).all()
