"""GPU parity of moe_quantize_mx against the oracle's MX quantizer:
bit-exact codes and scales (every finite bf16 value, wide-range fp32
values including subnormals, ragged row counts, both element formats)."""
import numpy as np
import pytest
import torch

from oracle import mx
from tests.gpu_util import log

pytestmark = pytest.mark.gpu


def _run(gpu_lib, v: np.ndarray, in_fmt: str, fmt: str):
    t = torch.from_numpy(v.astype(np.float32))
    t = (t.to(torch.bfloat16) if in_fmt == "bf16" else t).cuda()
    codes, scales = gpu_lib.quantize_mx(t, fmt)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def _oracle(v, fmt):
    el = "e4m3" if fmt == "mxfp8" else "e2m1"
    c, s = mx.quantize(v, el)
    if fmt == "mxfp4":
        c = mx.pack_fp4(c)
    return c, s


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_every_finite_bf16(gpu_lib, fmt):
    log(f"quantize every finite bf16 value, {fmt}")
    bits = np.arange(65536, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    v = v[np.isfinite(v)]
    v = v[np.random.default_rng(5).permutation(len(v))]
    v = v[: len(v) // 256 * 256].reshape(-1, 256)
    c, s = _run(gpu_lib, v, "bf16", fmt)
    oc, os_ = _oracle(v, fmt)
    assert np.array_equal(s, os_)
    assert np.array_equal(c, oc)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("rows,K", [(1, 32), (37, 7168), (129, 4096), (3, 96)])
def test_fp32_wide_range(gpu_lib, fmt, rows, K):
    log(f"quantize fp32 {rows}x{K} {fmt}")
    g = np.random.default_rng(rows * K)
    scale = np.exp2(g.integers(-140, 100, (rows, K // 32, 1)).astype(np.float64))
    v = (g.standard_normal((rows, K // 32, 32)) * scale).reshape(rows, K)
    v = v.astype(np.float32)
    v[0, :32] = 0.0                      # all-zero block
    if K >= 64:
        v[0, 32:64] = -0.0
    c, s = _run(gpu_lib, v, "fp32", fmt)
    oc, os_ = _oracle(v, fmt)
    assert np.array_equal(s, os_)
    assert np.array_equal(c, oc)


def test_halfway_and_saturation_values(gpu_lib):
    from tests.test_oracle_mx import _load_boundaries
    for fmt, amax, v, want in _load_boundaries():
        blk = np.zeros((1, 32), np.float32)
        blk[0, 0], blk[0, 1] = amax, v
        f = "mxfp8" if fmt == "e4m3" else "mxfp4"
        c, s = _run(gpu_lib, blk, "fp32", f)
        codes = mx.unpack_fp4(c) if f == "mxfp4" else c
        got = mx.dequantize(codes, s, fmt)[0, 1]
        assert got == np.float32(want), (fmt, amax, v, got, want)
