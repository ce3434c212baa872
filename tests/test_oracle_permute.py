"""Pins for the oracle's permutation maps, gather and summing un-permute.

Pinned against: one Python sort of (expert, token, slot) triples, the maps'
invariants (bijection onto live rows, counts summing to T*k, offsets an
exclusive scan of padded counts, stable order, padding marked -1), the
identity x_perm[row(t, j)] == x[t] bit for bit, un-permute of a k = 1
permute returning x, and quantize-then-permute equal to
permute-then-quantize.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import mx, permute as pm
from tests import brute


def _idx(seed, T, E, k):
    g = np.random.default_rng(seed)
    if T == 0:
        return np.zeros((0, k), np.int32)
    return np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("align", [1, 16, 32, 64, 128])
def test_matches_sorted_triples(align):
    idx = _idx(align, 50, 12, 4)
    got = pm.permute_maps(idx, 12, align)
    ref = brute.bf_permute(idx, 12, align)
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)


@settings(max_examples=50, deadline=None)
@given(seed=st.integers(0, 10 ** 6), T=st.integers(0, 40), E=st.integers(1, 20),
       align=st.sampled_from([1, 16, 32]), data=st.data())
def test_invariants(seed, T, E, align, data):
    k = data.draw(st.integers(1, E))
    idx = _idx(seed, T, E, k).reshape(T, k)
    counts, offsets, row_map, src = pm.permute_maps(idx, E, align)
    assert counts.sum() == T * k
    pc = (counts + align - 1) // align * align
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), pc)
    assert len(src) == pm.rows_bound(T, k, E, align)
    live = src >= 0
    assert live.sum() == T * k
    assert sorted(row_map.ravel().tolist()) == sorted(np.nonzero(live)[0].tolist())
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            r = row_map[t, j]
            assert offsets[e] <= r < offsets[e] + counts[e] and src[r] == t
    # stability: inside an expert, rows follow (t, j) order
    for e in range(E):
        seg = [(t, j) for t in range(T) for j in range(k) if idx[t, j] == e]
        assert [row_map[t, j] for t, j in seg] == list(range(offsets[e], offsets[e] + len(seg)))


def test_gather_identity_and_padding_zero():
    g = np.random.default_rng(1)
    idx = _idx(2, 30, 8, 3)
    x = g.standard_normal((30, 64)).astype(np.float32)
    _, offsets, row_map, src = pm.permute_maps(idx, 8, 16)
    xp = pm.permute_rows(x, src)
    for t in range(30):
        for j in range(3):
            assert np.array_equal(xp[row_map[t, j]].view(np.uint32), x[t].view(np.uint32))
    assert (xp[src < 0] == 0).all()


def test_unpermute_inverts_k1_and_sums_k():
    g = np.random.default_rng(3)
    x = g.standard_normal((25, 32)).astype(np.float32)
    idx = _idx(4, 25, 6, 1)
    _, _, rm, src = pm.permute_maps(idx, 6, 1)
    assert np.array_equal(pm.unpermute_sum(pm.permute_rows(x, src), rm).view(np.uint32), x.view(np.uint32))
    # k copies of bf16-valued rows sum exactly to k * x
    xb = (x.view(np.uint32) & 0xFFFF0000).view(np.float32)
    idx = _idx(5, 25, 6, 4)
    _, _, rm, src = pm.permute_maps(idx, 6, 32)
    assert np.array_equal(pm.unpermute_sum(pm.permute_rows(xb, src), rm), 4 * xb)


def test_quantize_commutes_with_permute():
    g = np.random.default_rng(6)
    x = g.standard_normal((20, 64)).astype(np.float32)
    idx = _idx(7, 20, 5, 2)
    _, _, _, src = pm.permute_maps(idx, 5, 1)
    c, s = mx.quantize(x, "e4m3")
    cp, sp = mx.quantize(pm.permute_rows(x, src), "e4m3")
    assert np.array_equal(pm.permute_rows(c, src), cp) and np.array_equal(pm.permute_rows(s, src), sp)


def test_empty_and_unused_experts():
    idx = np.zeros((0, 3), np.int32)
    counts, offsets, rm, src = pm.permute_maps(idx, 4, 16)
    assert counts.sum() == 0 and (offsets == 0).all() and len(src) == 4 * 15 and (src == -1).all()
    idx = np.array([[2, 0]], np.int32)
    counts, offsets, rm, src = pm.permute_maps(idx, 4, 1)
    assert list(counts) == [1, 0, 1, 0] and list(offsets) == [0, 1, 1, 2, 2]
    assert list(rm[0]) == [1, 0]
