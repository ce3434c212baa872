"""GPU parity of moe_permute against the oracle's maps and gather:
counts, offsets, row_map and src_row bit-exact for every alignment, ragged
and empty inputs, unused experts and skewed loads; gathered rows and scale
rows bit-exact with zero padding; repeated runs identical (no atomics)."""
import numpy as np
import pytest
import torch

from oracle import permute as pm
from tests.gpu_util import log

pytestmark = pytest.mark.gpu


def _idx(seed, T, E, k, skew=False):
    g = np.random.default_rng(seed)
    if T == 0:
        return np.zeros((0, k), np.int32)
    if skew:
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p[-2:] = 0
        p /= p.sum()
        rows = []
        for _ in range(T):
            rows.append(g.choice(E, k, replace=False, p=p))
        return np.array(rows, np.int32)
    return np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


def _permute(gpu_lib, idx, E, align, rows=None, scales=None):
    T, k = idx.shape
    bound = gpu_lib.moe_permute_rows_bound(T, k, E, align)
    i32 = dict(dtype=torch.int32, device="cuda")
    counts, offsets = torch.empty(E, **i32), torch.empty(E + 1, **i32)
    row_map, src = torch.empty((max(T, 1), k), **i32), torch.empty(max(bound, 1), **i32)
    ws = torch.empty(max(1, gpu_lib.moe_permute_workspace(T, k, E)), dtype=torch.uint8, device="cuda")
    idx_d = torch.from_numpy(idx).cuda() if T else None
    rows_out = torch.full((max(bound, 1), rows.shape[1]), 0x55, dtype=torch.uint8, device="cuda") if rows is not None else None
    sc_out = torch.full((max(bound, 1), scales.shape[1]), 0x55, dtype=torch.uint8, device="cuda") if scales is not None else None
    gpu_lib.moe_permute(idx_d, T, k, E, align,
                        None if rows is None else torch.from_numpy(rows).cuda(),
                        0 if rows is None else rows.shape[1],
                        None if scales is None else torch.from_numpy(scales).cuda(),
                        0 if scales is None else scales.shape[1],
                        counts, offsets, row_map if T else None, src, rows_out, sc_out, ws)
    torch.cuda.synchronize()
    out = [counts.cpu().numpy(), offsets.cpu().numpy(), row_map.cpu().numpy()[:T], src.cpu().numpy()[:bound]]
    if rows is not None:
        out.append(rows_out.cpu().numpy()[:bound])
    if scales is not None:
        out.append(sc_out.cpu().numpy()[:bound])
    return out


@pytest.mark.parametrize("T,E,k,align,skew", [
    (64, 16, 4, 1, False), (4096, 256, 8, 1, False), (16384, 256, 6, 1, False),
    (8192, 384, 6, 32, True), (300, 48, 6, 32, True), (1, 8, 3, 128, False), (1000, 3, 3, 16, False),
    (0, 12, 2, 32, False), (2049, 1024, 5, 64, True)])
def test_maps_bit_exact(gpu_lib, T, E, k, align, skew):
    log(f"permute maps T={T} E={E} k={k} align={align} skew={skew}")
    idx = _idx(T * 7 + E, T, E, k, skew)
    got = _permute(gpu_lib, idx, E, align)
    ref = pm.permute_maps(idx, E, align)
    for name, a, b in zip(["counts", "offsets", "row_map", "src_row"], got, ref):
        assert np.array_equal(a, b), name
    again = _permute(gpu_lib, idx, E, align)
    for a, b in zip(got, again):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("row_bytes,scale_bytes,align", [(14336, 224, 1), (16, 1, 32), (1024, 12, 16)])
def test_rows_and_scales_gather(gpu_lib, row_bytes, scale_bytes, align):
    log(f"permute gather row_bytes={row_bytes} scale_bytes={scale_bytes} align={align}")
    T, E, k = 150, 20, 4
    g = np.random.default_rng(row_bytes)
    idx = _idx(9, T, E, k)
    rows = g.integers(0, 256, (T, row_bytes), dtype=np.uint8)
    scales = g.integers(0, 256, (T, scale_bytes), dtype=np.uint8)
    c, o, rm, src, rout, sout = _permute(gpu_lib, idx, E, align, rows, scales)
    _, _, _, osrc = pm.permute_maps(idx, E, align)
    assert np.array_equal(rout, pm.permute_rows(rows, osrc))
    assert np.array_equal(sout, pm.permute_rows(scales, osrc))
    for t in range(T):
        for j in range(k):
            assert np.array_equal(rout[rm[t, j]], rows[t])
