"""Pins of the oracle's top-k routing and cache lookup (CPU).

* top-k against brute-force enumeration of all k-subsets on tiny inputs
  (the chosen set maximises the sum of ranks under the stated total order)
  and against numpy's stable argsort on larger ones
* ties, -0.0/+0.0, NaN, all-equal logits, k = E
* weights: sum to 1, k = 1 gives 1, equal logits give 1/k, ratios equal
  exp of logit differences (scipy's softmax on the chosen logits)
* lookup: hits + misses = the chosen multiset; misses sorted and distinct
"""
import itertools

import numpy as np
import pytest
import scipy.special

import oracle


def _brute_topk(row, k):
    """The k-subset that is lexicographically best under (value desc,
    index asc), found by enumerating every subset."""
    E = len(row)
    key = [(-(-np.inf if v != v else v + 0.0), e) for e, v in enumerate(row)]
    best = None
    for comb in itertools.combinations(range(E), k):
        ks = sorted(key[e] for e in comb)
        if best is None or ks < best:
            best = ks
    return [e for _, e in best]


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    E, k = 9, 4
    logits = rng.integers(-3, 4, size=(5, E)).astype(np.float32)  # many ties
    logits[0, 2] = -0.0
    logits[0, 5] = 0.0
    logits[1, 3] = np.nan
    logits[2, :] = np.nan
    idx, w = oracle.route_topk(logits, k)
    for t in range(logits.shape[0]):
        assert list(idx[t]) == _brute_topk(logits[t], k)


def test_topk_matches_stable_argsort():
    rng = np.random.default_rng(7)
    logits = rng.normal(0, 1.5, size=(16, 512)).astype(np.float32)
    idx, w = oracle.route_topk(logits, 10)
    ref = np.argsort(-logits, axis=1, kind="stable")[:, :10]
    np.testing.assert_array_equal(idx, ref)
    chosen = np.take_along_axis(logits, ref, 1).astype(np.float64)
    np.testing.assert_allclose(w, scipy.special.softmax(chosen, axis=1), rtol=1e-13)


def test_topk_special_cases():
    E = 16
    eq = np.zeros((1, E), np.float32)
    idx, w = oracle.route_topk(eq, 5)
    assert list(idx[0]) == [0, 1, 2, 3, 4]
    np.testing.assert_allclose(w[0], 0.2, rtol=0, atol=1e-15)
    rng = np.random.default_rng(1)
    l = rng.normal(size=(3, E)).astype(np.float32)
    idx, w = oracle.route_topk(l, E)                   # k = E: full order
    for t in range(3):
        assert sorted(idx[t]) == list(range(E))
        assert np.all(np.diff(l[t, idx[t]]) <= 0)
    idx, w = oracle.route_topk(l, 1)
    np.testing.assert_array_equal(w, 1.0)
    np.testing.assert_array_equal(idx[:, 0], np.argmax(l, 1))
    # infinities: +inf entries share the weight, -inf ones get none
    l2 = np.array([[1.0, np.inf, 3.0, np.inf, -np.inf]], np.float32)
    idx, w = oracle.route_topk(l2, 3)
    assert list(idx[0]) == [1, 3, 2]
    np.testing.assert_array_equal(w[0], [0.5, 0.5, 0.0])
    l3 = np.full((1, 4), -np.inf, np.float32)
    idx, w = oracle.route_topk(l3, 2)
    assert list(idx[0]) == [0, 1]
    np.testing.assert_array_equal(w[0], [0.5, 0.5])


@pytest.mark.parametrize("seed", range(3))
def test_weights_sum_to_one(seed):
    rng = np.random.default_rng(seed)
    l = rng.normal(0, 3.0, size=(32, 64)).astype(np.float32)
    _, w = oracle.route_topk(l, 7)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)
    assert np.all(w[:, :-1] >= w[:, 1:])


def test_lookup_partition():
    rng = np.random.default_rng(3)
    E, T, k = 40, 4, 6
    table = np.full(E, -1, np.int32)
    res = rng.choice(E, 15, replace=False)
    table[res] = rng.permutation(15)
    l = rng.normal(size=(T, E)).astype(np.float32)
    idx, _ = oracle.route_topk(l, k)
    slot, miss_e, miss_p, n = oracle.cache_lookup(idx, table)
    assert n[0] == len(miss_e) and n[1] == len(miss_p)
    hits = [(t, i) for t in range(T) for i in range(k) if slot[t, i] >= 0]
    misses = [(p // k, p % k) for p in miss_p]
    assert sorted(hits + misses) == [(t, i) for t in range(T) for i in range(k)]
    for t, i in hits:
        assert table[idx[t, i]] == slot[t, i] >= 0
    for t, i in misses:
        assert table[idx[t, i]] == -1
    assert list(miss_e) == sorted(set(int(idx[t, i]) for t, i in misses))
    keys = [(idx[p // k, p % k], p // k, p % k) for p in miss_p]
    assert keys == sorted(keys)


def test_lookup_all_resident_and_none_resident():
    idx = np.array([[3, 1, 2]], np.int32)
    slot, me, mp, n = oracle.cache_lookup(idx, np.arange(8, dtype=np.int32)[::-1])
    assert list(slot[0]) == [4, 6, 5] and list(n) == [0, 0]
    slot, me, mp, n = oracle.cache_lookup(idx, np.full(8, -1, np.int32))
    assert list(me) == [1, 2, 3] and list(mp) == [1, 2, 0] and list(n) == [3, 3]
