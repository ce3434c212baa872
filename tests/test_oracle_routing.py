"""Pins for the oracle's router: logits, sigmoid scores, grouped top-k and
combine weights.

Pinned against: scalar brute force with Python tuple sorts, the
definition's invariants (exactly k distinct experts inside the kept groups,
every kept group scoring at least every dropped one, no unpicked candidate
above a picked one), library special cases (n_group = 1 is plain top-k,
checked with heapq), closed forms (one-hot inputs, sigma(0) = 1/2, equal
scores) and planted mistakes that the pins must catch.
"""
import heapq
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import routing as rt
from tests import brute


def _draw(seed, T, E, scale=1.0, bias=0.1):
    g = np.random.default_rng(seed)
    logits = (g.standard_normal((T, E)) * scale).astype(np.float32)
    b = g.uniform(-bias, bias, E).astype(np.float32)
    return logits, b


def test_logits_closed_forms():
    g = np.random.default_rng(0)
    w = g.standard_normal((16, 64)).astype(np.float32)
    x = np.eye(64, dtype=np.float32)[:5]
    assert np.array_equal(rt.router_logits(x, w), w[:, :5].T)
    # brute force with exact summation, then one rounding
    x = g.standard_normal((3, 64)).astype(np.float32)
    ref = np.array([[np.float32(math.fsum(float(a) * float(b) for a, b in zip(x[t], w[e])))
                     for e in range(16)] for t in range(3)])
    got = rt.router_logits(x, w)
    assert np.max(np.abs(got.view(np.int32) - ref.view(np.int32))) <= 1


def test_sigmoid_closed_forms():
    s = rt.sigmoid_scores(np.array([0.0, math.log(3.0), -math.log(3.0), 100.0, -100.0], np.float32))
    assert s[0] == 0.5
    assert abs(s[1] - 0.75) <= 2 ** -24 and abs(s[2] - 0.25) <= 2 ** -25
    assert s[3] == 1.0 and 0 < s[4] < 1e-40


@pytest.mark.parametrize("E,n_group,topk_group,k", [
    (16, 4, 2, 4), (32, 8, 4, 8), (24, 6, 3, 5), (8, 4, 2, 3), (16, 1, 1, 6), (12, 6, 6, 12)])
def test_matches_brute_force(E, n_group, topk_group, k):
    logits, b = _draw(E * 7 + k, 64, E)
    idx, w, _, _ = rt.route(logits, b, n_group, topk_group, k, 2.5)
    bidx, bw = brute.bf_route(logits, b, n_group, topk_group, k, 2.5)
    assert np.array_equal(idx, bidx)
    assert np.array_equal(w, bw)


def check_invariants(logits, b, n_group, topk_group, k, idx):
    s = rt.sigmoid_scores(logits)
    sel = (s + b).astype(np.float32)
    T, E = logits.shape
    G = E // n_group
    for t in range(T):
        row = list(idx[t])
        assert len(set(row)) == k
        assert all(sel[t, row[j]] >= sel[t, row[j + 1]] for j in range(k - 1))
        groups = {e // G for e in row}
        assert len(groups) <= topk_group
        if n_group > 1:
            gs = []
            for q in range(n_group):
                top = sorted(sel[t, q * G:(q + 1) * G], reverse=True)
                gs.append(np.float32(top[0] + top[1]))
            order = sorted(range(n_group), key=lambda q: (-gs[q], q))
            kept = set(order[:topk_group])
            assert groups <= kept
            cand = [e for e in range(E) if e // G in kept]
        else:
            cand = list(range(E))
        lo = min(sel[t, e] for e in row)
        for e in cand:
            if e not in row:
                assert sel[t, e] < lo or (sel[t, e] == lo and e > max(x for x in row if sel[t, x] == lo))


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 10 ** 6), T=st.integers(1, 20), n_group=st.sampled_from([1, 2, 4, 8]),
       gsize=st.sampled_from([2, 3, 4, 8]), data=st.data())
def test_invariants_random(seed, T, n_group, gsize, data):
    E = n_group * gsize
    topk_group = data.draw(st.integers(1, n_group))
    k = data.draw(st.integers(1, topk_group * gsize))
    logits, b = _draw(seed, T, E, scale=data.draw(st.sampled_from([0.01, 1.0, 8.0])))
    idx, w, _, _ = rt.route(logits, b, n_group, topk_group, k, 1.0)
    check_invariants(logits, b, n_group, topk_group, k, idx)
    assert (w > 0).all()


def test_ties_go_to_lower_index():
    logits = np.zeros((1, 8), np.float32)
    b = np.zeros(8, np.float32)
    idx, w, _, _ = rt.route(logits, b, 4, 2, 3, 1.0)
    assert list(idx[0]) == [0, 1, 2]
    bidx, _ = brute.bf_route(logits, b, 4, 2, 3, 1.0)
    assert list(bidx[0]) == [0, 1, 2]


def test_plain_topk_equals_heapq():
    logits, b = _draw(3, 50, 40)
    idx, _, s, sel = rt.route(logits, b, 1, 1, 6, 1.0)
    for t in range(50):
        ref = heapq.nlargest(6, range(40), key=lambda e: (sel[t, e], -e))
        assert list(idx[t]) == ref


def test_no_bias_plain_topk_follows_logits():
    logits, _ = _draw(4, 30, 32, scale=2.0)
    idx, _, _, _ = rt.route(logits, np.zeros(32, np.float32), 1, 1, 4, 1.0)
    ref = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :4]
    assert np.array_equal(idx, ref)


def test_weights_closed_forms():
    logits, b = _draw(5, 40, 16)
    idx, w, s, _ = rt.route(logits, b, 4, 2, 4, 2.5)
    tot = w.astype(np.float64).sum(1)
    assert np.all(np.abs(tot - 2.5) <= 4 * 2.5 * 2 ** -23)
    # equal scores: every weight is scale / k exactly (k a power of two)
    idx, w, _, _ = rt.route(np.zeros((3, 16), np.float32), np.zeros(16, np.float32), 4, 2, 4, 2.5)
    assert (w == np.float32(2.5 / 4)).all()
    # one expert, k = 1: the weight is the routed scale exactly
    idx, w, _, _ = rt.route(np.array([[0.3], [-4.0]], np.float32), np.zeros(1, np.float32), 1, 1, 1, 2.5)
    assert (idx == 0).all() and (w == np.float32(2.5)).all()


def test_bias_is_for_selection_only():
    logits, _ = _draw(6, 20, 16)
    b = np.zeros(16, np.float32)
    b[3] = 5.0                     # forces expert 3 into every selection
    idx, w, s, _ = rt.route(logits, b, 1, 1, 2, 1.0)
    assert (idx[:, 0] == 3).all()
    # its weight still uses the unbiased score
    other = idx[:, 1]
    sc = rt.sigmoid_scores(logits)
    ref = sc[np.arange(20), 3] / (sc[np.arange(20), 3] + sc[np.arange(20), other])
    assert np.allclose(w[:, 0], ref, rtol=2e-7)


def test_planted_mistakes_are_caught(monkeypatch):
    """Each plausible slip in the oracle fails the brute-force pin."""
    logits, b = _draw(7, 64, 32, scale=1.0, bias=0.5)
    bidx, bw = brute.bf_route(logits, b, 8, 4, 8, 2.5)

    def differs():
        idx, w, _, _ = rt.route(logits, b, 8, 4, 8, 2.5)
        return not (np.array_equal(idx, bidx) and np.array_equal(w, bw))

    assert not differs()
    orig_gs = rt.group_scores
    monkeypatch.setattr(rt, "group_scores", lambda sel, n: (-np.sort(-sel.reshape(sel.shape[0], n, -1), 2)[:, :, 0]))
    assert differs(), "max-per-group scoring must be caught"
    monkeypatch.setattr(rt, "group_scores", orig_gs)
    orig_sel = rt.selection_scores
    monkeypatch.setattr(rt, "selection_scores", lambda s, bias: s)
    assert differs(), "dropping the selection bias must be caught"
    monkeypatch.setattr(rt, "selection_scores", orig_sel)
    orig_cw = rt.combine_weights
    monkeypatch.setattr(rt, "combine_weights",
                        lambda s, idx, sc: orig_cw(orig_sel(s, b), idx, sc))
    assert differs(), "weighting by biased scores must be caught"
    monkeypatch.setattr(rt, "combine_weights", orig_cw)
    assert not differs()
