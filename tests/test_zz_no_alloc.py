"""moe_permute_noalloc (the permute for callers that cannot allocate)
against moe_permute on the same inputs: every map and the gathered rows bit
for bit, on two calls in a row, the second with a smaller input, so the
second runs on the array the first left behind. Also the size limit."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_sigmoid_amd as moe
from tests.gpu_util import log

pytestmark = pytest.mark.gpu


def _run(fn, idx, T, k, E, align, x):
    dev = dict(dtype=torch.int32, device="cuda")
    bound = moe.moe_permute_rows_bound(T, k, E, align)
    counts = torch.full((E,), -7, **dev)
    offsets = torch.full((E + 1,), -7, **dev)
    row_map = torch.full((T, k), -7, **dev)
    src = torch.full((max(1, bound),), -7, **dev)
    rows = torch.full((max(1, bound), x.shape[1]), 99, dtype=torch.uint8, device="cuda")
    if fn == "ws":
        ws = torch.empty(max(1, moe.moe_permute_workspace(T, k, E)), dtype=torch.uint8, device="cuda")
        moe.moe_permute(idx, T, k, E, align, x, x.shape[1], None, 0, counts, offsets, row_map, src,
                        rows, None, ws)
    else:
        moe.moe_permute_noalloc(idx, T, k, E, align, x, x.shape[1], None, 0, counts, offsets,
                                row_map, src, rows, None)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (counts, offsets, row_map, src[:bound], rows[:bound])]


@pytest.mark.parametrize("T,k,E,align", [(16384, 6, 256, 1), (4096, 8, 256, 32), (300, 6, 48, 16)])
def test_noalloc_matches_workspace_call(gpu_lib, T, k, E, align):
    assert moe.moe_permute_workspace(T, k, E) <= moe.moe_permute_noalloc_max_bytes()
    g = np.random.default_rng(T + E)
    for call, n in enumerate((T, T // 3 + 1)):       # the second call is smaller
        log(f"permute_noalloc call {call}: T={n} k={k} E={E} align={align}")
        idx_h = np.stack([g.permutation(E)[:k] for _ in range(n)]).astype(np.int32)
        idx = torch.from_numpy(idx_h).cuda()
        x = torch.from_numpy(g.integers(0, 255, (n, 64), dtype=np.uint8)).cuda()
        ref = _run("ws", idx, n, k, E, align, x)
        got = _run("noalloc", idx, n, k, E, align, x)
        for name, a, b in zip(["counts", "offsets", "row_map", "src_row", "rows"], got, ref):
            assert np.array_equal(a, b), (call, name)


def test_noalloc_rejects_oversize(gpu_lib):
    T, k, E = 1 << 16, 8, 1024          # 512 chunks x 1024 experts x 4 B = 2 MiB > 1 MiB
    assert moe.moe_permute_workspace(T, k, E) > moe.moe_permute_noalloc_max_bytes()
    A = torch.empty(16, dtype=torch.int32, device="cuda")
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_permute_noalloc(A, T, k, E, 1, None, 0, None, 0, A, A, A, A, None, None)
    assert ei.value.status == -4 and "1 MiB" in str(ei.value)
