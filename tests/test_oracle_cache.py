"""Pins of the oracle's cache admission and eviction (CPU).

* counting equals numpy's bincount
* with no swap limit the planned cache is the best one: brute force over
  every cache of the same size on tiny inputs gives the largest total count,
  and among those the plan changes the fewest slots
* a swap limit m gives the first m swaps of the unlimited plan, and a second
  plan finishes the rest
* every swap strictly raises the slot's count; the shared slot, experts with
  no host copy and unused experts are never admitted
* decay is a right shift; after commit the two tables are inverse
"""
import itertools

import numpy as np
import pytest

import oracle


def _state(rng, E, n_slots, shared_slot, n_res, host_missing=()):
    eos = np.full(n_slots, -1, np.int32)
    res = rng.choice(E, n_res, replace=False)
    free = [s for s in range(n_slots) if s != shared_slot]
    rng.shuffle(free)
    for s, e in zip(free, res):
        eos[s] = e
    if shared_slot >= 0:
        eos[shared_slot] = E
    soe = np.full(E, -1, np.int32)
    for s, e in enumerate(eos):
        if 0 <= e < E:
            soe[e] = s
    hs = rng.permutation(E).astype(np.int32)
    for e in host_missing:
        hs[e] = -1
    return soe, eos, hs


def test_count_is_bincount():
    rng = np.random.default_rng(0)
    E = 300
    idx = np.stack([rng.choice(E, 10, replace=False) for _ in range(37)])
    c0 = rng.integers(0, 1000, E).astype(np.uint32)
    got = oracle.cache_count(c0, idx)
    np.testing.assert_array_equal(got, c0 + np.bincount(idx.reshape(-1), minlength=E))
    # wraps at 2^32 like a uint32 counter
    c1 = np.full(E, 0xFFFFFFFF, np.uint32)
    got = oracle.cache_count(c1, idx[:1])
    assert all(got[e] == 0 for e in idx[0])


def _resident(eos, shared_slot, E):
    return {int(e) for s, e in enumerate(eos) if s != shared_slot and 0 <= e < E}


@pytest.mark.parametrize("seed", range(12))
def test_unlimited_plan_is_best_cache(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(4, 9))
    n_slots = int(rng.integers(2, 6))
    shared_slot = int(rng.integers(-1, n_slots)) if seed % 2 else -1
    cap = n_slots - (1 if shared_slot >= 0 else 0)
    n_res = int(rng.integers(0, min(cap, E) + 1))
    missing = [int(e) for e in rng.choice(E, int(rng.integers(0, 2)), replace=False)]
    soe, eos, hs = _state(rng, E, n_slots, shared_slot, n_res, missing)
    cnt = rng.integers(0, 4, E).astype(np.uint32)       # small range: many ties
    new_cnt, soe2, eos2, swaps = oracle.cache_plan(cnt, soe, eos, shared_slot, hs, E, 99, 0)
    np.testing.assert_array_equal(new_cnt, cnt)
    soe3 = oracle.cache_commit(soe2, swaps)
    before = _resident(eos, shared_slot, E)
    after = _resident(eos2, shared_slot, E)
    # brute force: caches of at most cap experts, built from current residents
    # and admissible experts (a host copy and a count above 0)
    admissible = {e for e in range(E) if hs[e] >= 0 and cnt[e] > 0}
    pool = sorted(before | admissible)
    best = None
    for r in range(0, min(cap, len(pool)) + 1):
        for S in itertools.combinations(pool, r):
            S = set(S)
            key = (int(sum(int(cnt[e]) for e in S)), -len(S - before))
            best = key if best is None or key > best else best
    got = (int(sum(int(cnt[e]) for e in after)), -len(after - before))
    assert got == best, (got, best)
    assert len(swaps) == len(after - before)
    # tables consistent after commit; shared slot untouched
    for s, e in enumerate(eos2):
        if s == shared_slot:
            assert e == eos[s]
        elif e >= 0:
            assert soe3[e] == s
    assert {e for e in range(E) if soe3[e] >= 0} == after
    for s, old, e, h in swaps:
        assert cnt[e] > (cnt[old] if old >= 0 else -1)
        assert h == hs[e] and e in admissible and s != shared_slot


def test_swap_limit_is_prefix_and_resumes():
    rng = np.random.default_rng(7)
    E, n_slots, shared_slot = 200, 41, 17
    soe, eos, hs = _state(rng, E, n_slots, shared_slot, 30, host_missing=(3, 5))
    cnt = rng.integers(0, 50, E).astype(np.uint32)
    _, soe_u, eos_u, sw_u = oracle.cache_plan(cnt, soe, eos, shared_slot, hs, E, 1000, 0)
    assert len(sw_u) > 6
    c1, soe1, eos1, sw1 = oracle.cache_plan(cnt, soe, eos, shared_slot, hs, E, 6, 0)
    assert sw1 == sw_u[:6]
    soe1 = oracle.cache_commit(soe1, sw1)
    _, soe2, eos2, sw2 = oracle.cache_plan(c1, soe1, eos1, shared_slot, hs, E, 1000, 0)
    assert _resident(eos2, shared_slot, E) == _resident(eos_u, shared_slot, E)
    assert len(sw1) + len(sw2) == len(sw_u)
    assert 3 not in _resident(eos2, shared_slot, E) or soe[3] >= 0


def test_decay_and_no_admission_of_unused():
    rng = np.random.default_rng(8)
    E, n_slots = 64, 20
    soe, eos, hs = _state(rng, E, n_slots, -1, 0)
    cnt = np.zeros(E, np.uint32)
    cnt[[3, 9, 11]] = [7, 1, 12]
    new, soe2, eos2, sw = oracle.cache_plan(cnt, soe, eos, -1, hs, E, 99, 2)
    np.testing.assert_array_equal(new, cnt >> 2)
    assert [e for _, _, e, _ in sw] == [11, 3, 9]          # by count, only used experts
    assert [s for s, _, _, _ in sw] == [0, 1, 2]           # empty slots in slot order
    assert (eos2[3:] == -1).all()
    # the newcomers are not yet visible
    assert (soe2 == -1).all()
