"""Pins of the oracle's routing and dispatch (CPU only).

Routing is checked against a brute-force full ordering, scipy's softmax and the
special cases top_k = 1 (weight exactly 1) and top_k = E (the full softmax);
the dispatch permutation against numpy's stable argsort.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle


def _brute_route(logits, k):
    T, E = logits.shape
    ids = np.zeros((T, k), np.int64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))
        ids[t] = order[:k]
    p = softmax(logits.astype(np.float64), axis=1)
    sel = np.take_along_axis(p, ids, axis=1)
    w = sel / sel.sum(axis=1, keepdims=True)
    return ids, w


def _ulp_diff(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (33, 384, 6), (20, 128, 3), (5, 1024, 8), (3, 7, 7)])
def test_route_matches_brute_force(T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = oracle.route(lg, k)
    bids, bw = _brute_route(lg, k)
    assert np.array_equal(ids, bids)
    assert _ulp_diff(w, bw.astype(np.float32)).max() <= 1


def test_route_ties_take_lower_index():
    lg = np.zeros((2, 8), np.float32)
    lg[0, [5, 2, 7]] = 1.0
    lg[1, :] = 3.0
    ids, w = oracle.route(lg, 3)
    assert ids[0].tolist() == [2, 5, 7]
    assert ids[1].tolist() == [0, 1, 2]
    assert np.all(w[1] == np.float32(1.0 / 3.0))


def test_route_top1_weight_is_one():
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((50, 384)).astype(np.float32)
    ids, w = oracle.route(lg, 1)
    assert np.all(w == 1.0)
    assert np.array_equal(ids[:, 0], np.argmax(lg, axis=1))


def test_route_all_experts_is_softmax():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((40, 8)).astype(np.float32) * 3
    ids, w = oracle.route(lg, 8)
    p = softmax(lg.astype(np.float64), axis=1)
    assert np.array_equal(ids, np.argsort(-lg, axis=1, kind="stable"))
    assert _ulp_diff(w, np.take_along_axis(p, ids, 1).astype(np.float32)).max() <= 1


def test_route_weights_sum_to_one():
    rng = np.random.default_rng(3)
    lg = (rng.standard_normal((200, 384)) * 2).astype(np.float32)
    _, w = oracle.route(lg, 6)
    s = w.astype(np.float64).sum(axis=1)
    assert np.abs(s - 1).max() <= 4 * 2.0 ** -24


def test_route_extreme_logits_are_finite():
    lg = np.array([[80.0, -80.0, 0.0, 79.0], [-1e30, -1e30, 1e30, 0.0]], np.float32)
    ids, w = oracle.route(lg, 2)
    assert ids.tolist() == [[0, 3], [2, 3]]
    assert np.all(np.isfinite(w)) and np.allclose(w.sum(1), 1)


@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (64, 384, 6), (1000, 384, 6), (7, 128, 3), (1, 4, 4)])
def test_sort_matches_stable_argsort(T, E, k):
    rng = np.random.default_rng(T + E)
    ids, _ = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    counts, offsets, perm = oracle.sort(ids, E)
    flat = ids.reshape(-1)
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and np.array_equal(offsets[1:], np.cumsum(counts))
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))


def test_sort_invariants_skewed():
    from quantized_moe_expert_softmax_amd import synth
    lg = synth.router_logits(4096, 384, 9, skewed=True)
    ids, _ = oracle.route(lg, 6)
    counts, offsets, perm = oracle.sort(ids, 384)
    flat = ids.reshape(-1)
    assert counts.sum() == flat.size
    assert np.array_equal(np.sort(perm), np.arange(flat.size))
    for e in range(384):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)
    # the skew leaves experts empty and loads some far above the mean
    assert (counts == 0).sum() > 0 and counts.max() > 4 * counts.mean()
