"""Pins of the oracle's expert FFN, layer and combine (CPU).

* closed form: one-hot activations on constant-block experts
* silu(z) - silu(-z) = z, silu against scipy's expit
* k = E reproduces the plain softmax mixture of every expert (scipy softmax)
* the sparse top-k layer equals a brute-force dense evaluation of all E
  experts followed by selection
* combine is linear in the rows; a one-hot weight selects one row
* hits-only partial + the missed experts = the full layer
* two tiers (GPU cache + host copy): with every miss run it is the dense
  brute-force layer; raising the rank limit by one adds exactly the missed
  terms of that rank; a rank limit of 0 leaves the hits-only layer; the host
  slot order does not matter; an expert in neither tier adds nothing
* verify: T tokens at once equal T separate one-token layers
"""
import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth


def _unpack_all(slots, fmt, d, f):
    return [oracle.unpack_expert(s, fmt, d, f) for s in slots]


def test_silu_identities():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=0, atol=1e-13)
    np.testing.assert_allclose(oracle.silu(z), z * scipy.special.expit(z), rtol=1e-15, atol=1e-300)
    assert oracle.silu(0.0) == 0.0


def test_ffn_closed_form_one_hot():
    """Constant blocks quantize exactly (scale 0, min = the value)."""
    d, f = 64, 32
    a = (np.arange(f) % 5 - 2) / 4.0             # gate row j constant a_j
    b = (np.arange(f) % 3 + 1) / 8.0             # up row j constant b_j
    c = (np.arange(d) % 7 - 3) / 16.0            # down row r constant c_r
    Wg = torch.tensor(np.repeat(a[:, None], d, 1), dtype=torch.float32)
    Wu = torch.tensor(np.repeat(b[:, None], d, 1), dtype=torch.float32)
    Wd = torch.tensor(np.repeat(c[:, None], f, 1), dtype=torch.float32)
    G = torch.stack([Wg, Wu], 1).reshape(1, 2 * f, d)
    slot = synth.pack_expert_slots(G, Wd.unsqueeze(0), synth.FMT_Q2SM)[0].numpy()
    W = oracle.unpack_expert(slot, oracle.FMT_Q2SM, d, f)
    for col in (0, 17, 63):
        x = np.zeros((1, d))
        x[0, col] = 1.0
        o = oracle.expert_ffn(x, *W)[0]
        h = a * scipy.special.expit(a) * b
        np.testing.assert_allclose(o, c * h.sum(), rtol=1e-14, atol=1e-15)
    # x = 0 gives no change
    assert not oracle.expert_ffn(np.zeros((1, d)), *W).any()


def _tiny_layer(E=8, d=64, f=32, fmt=synth.FMT_Q2SM, seed=5, shared=True):
    gen = torch.Generator().manual_seed(seed)
    n = E + (1 if shared else 0)
    G = torch.randn(n, 2 * f, d, generator=gen) * 0.05
    D = torch.randn(n, d, f, generator=gen) * 0.05
    slots = synth.pack_expert_slots(G, D, fmt).numpy()
    W = _unpack_all(slots, fmt, d, f)
    return W[:E], (W[E] if shared else None)


def test_k_equals_E_is_softmax_mixture():
    E, d, f = 8, 64, 32
    W, Wsh = _tiny_layer(E, d, f, shared=False)
    rng = np.random.default_rng(0)
    x = rng.normal(size=(3, d))
    logits = rng.normal(size=(3, E)).astype(np.float32)
    idx, w = oracle.route_topk(logits, E)
    y = oracle.layer_decode(x, idx, idx, w, lambda s: W[s], None, hits_only=True)
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)          # [T,E]
    outs = np.stack([oracle.expert_ffn(x, *W[e]) for e in range(E)], 1)   # [T,E,d]
    ref = x + np.einsum("te,ted->td", p, outs)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("k", [1, 3, 8])
def test_sparse_equals_dense_brute_force(k):
    E, d, f = 8, 64, 32
    W, Wsh = _tiny_layer(E, d, f, shared=True)
    rng = np.random.default_rng(k)
    x = rng.normal(size=(4, d))
    logits = rng.normal(size=(4, E)).astype(np.float32)
    idx, w = oracle.route_topk(logits, k)
    table = np.arange(E, dtype=np.int32)
    slot, _, _, _ = oracle.cache_lookup(idx, table)
    allW = W + [Wsh]
    y = oracle.layer_decode(x, idx, slot, w, lambda s: allW[s], E)
    ref = oracle.layer_dense_mixture(x, logits, W, k, Wsh)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_partial_plus_misses_is_full():
    E, d, f, k = 12, 64, 32, 4
    W, Wsh = _tiny_layer(E, d, f, shared=True)
    rng = np.random.default_rng(9)
    x = rng.normal(size=(3, d))
    logits = rng.normal(size=(3, E)).astype(np.float32)
    idx, w = oracle.route_topk(logits, k)
    resident = [1, 4, 5, 7, 10]
    table = np.full(E, -1, np.int32)
    table[resident] = np.arange(len(resident))
    slots_W = [W[e] for e in resident] + [Wsh]
    shared_slot = len(resident)
    slot, miss_e, miss_p, n = oracle.cache_lookup(idx, table)
    part = oracle.layer_decode(x, idx, slot, w, lambda s: slots_W[s], shared_slot)
    full = part.copy()
    for p in miss_p:
        t, i = divmod(int(p), k)
        full[t] += w[t, i] * oracle.expert_ffn(x[t:t + 1], *W[idx[t, i]])[0]
    ref = oracle.layer_dense_mixture(x, logits, W, k, Wsh)
    np.testing.assert_allclose(full, ref, rtol=1e-12, atol=1e-13)
    assert n[1] > 0 and n[1] < 3 * k


def _two_tier_case(seed=11, E=16, d=64, f=32, k=5, T=4):
    W, Wsh = _tiny_layer(E, d, f, shared=True, seed=seed)
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(T, d))
    logits = rng.normal(size=(T, E)).astype(np.float32)
    idx, w = oracle.route_topk(logits, k)
    resident = [0, 3, 4, 9, 12, 13]
    table = np.full(E, -1, np.int32)
    table[resident] = np.arange(len(resident))
    gpu_W = [W[e] for e in resident] + [Wsh]
    host_order = rng.permutation(E)              # host slot h holds expert host_order[h]
    host_slot = np.empty(E, np.int32)
    host_slot[host_order] = np.arange(E)
    host_W = [W[e] for e in host_order]
    slot, _, miss_p, _ = oracle.cache_lookup(idx, table)
    return W, Wsh, x, logits, idx, w, slot, gpu_W, len(resident), host_slot, host_W, miss_p


def test_two_tiers_full_is_dense():
    W, Wsh, x, logits, idx, w, slot, gpu_W, sh, host_slot, host_W, miss_p = _two_tier_case()
    assert len(miss_p) > 0
    y = oracle.layer_decode_tiers(x, idx, w, slot, lambda s: gpu_W[s], sh, host_slot,
                                  lambda h: host_W[h])
    ref = oracle.layer_dense_mixture(x, logits, W, idx.shape[1], Wsh)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_two_tiers_rank_limit():
    W, Wsh, x, logits, idx, w, slot, gpu_W, sh, host_slot, host_W, miss_p = _two_tier_case(seed=12)
    T, k = idx.shape
    ys = [oracle.layer_decode_tiers(x, idx, w, slot, lambda s: gpu_W[s], sh, host_slot,
                                    lambda h: host_W[h], max_rank=r) for r in range(k + 1)]
    # rank limit 0: the hits-only layer, whatever the host tier holds
    part = oracle.layer_decode(x, idx, slot, w, lambda s: gpu_W[s], sh)
    np.testing.assert_array_equal(ys[0], part)
    zero_W = [tuple(np.zeros_like(m) for m in Wt) for Wt in host_W]
    y0z = oracle.layer_decode_tiers(x, idx, w, slot, lambda s: gpu_W[s], sh, host_slot,
                                    lambda h: zero_W[h], max_rank=0)
    np.testing.assert_array_equal(y0z, part)
    # each step of the limit adds the missed terms of that rank, nothing else
    for r in range(1, k + 1):
        for t in range(T):
            want = np.zeros(x.shape[1])
            if slot[t, r - 1] < 0:
                want = w[t, r - 1] * oracle.expert_ffn(x[t:t + 1], *W[idx[t, r - 1]])[0]
            np.testing.assert_allclose(ys[r][t] - ys[r - 1][t], want, rtol=1e-9, atol=1e-12)
    np.testing.assert_array_equal(ys[k], oracle.layer_decode_tiers(
        x, idx, w, slot, lambda s: gpu_W[s], sh, host_slot, lambda h: host_W[h]))


def test_two_tiers_host_order_and_absent():
    W, Wsh, x, logits, idx, w, slot, gpu_W, sh, host_slot, host_W, miss_p = _two_tier_case(seed=13)
    T, k = idx.shape
    E = len(W)
    full = oracle.layer_decode_tiers(x, idx, w, slot, lambda s: gpu_W[s], sh, host_slot,
                                     lambda h: host_W[h])
    # identity host order gives the same result
    same = oracle.layer_decode_tiers(x, idx, w, slot, lambda s: gpu_W[s], sh,
                                     np.arange(E, dtype=np.int32), lambda h: W[h])
    np.testing.assert_allclose(same, full, rtol=1e-13, atol=1e-14)
    # a missed expert absent from the host tier drops exactly its terms
    p = int(miss_p[0])
    e = int(idx.reshape(-1)[p])
    hs = host_slot.copy()
    hs[e] = -1
    got = oracle.layer_decode_tiers(x, idx, w, slot, lambda s: gpu_W[s], sh, hs,
                                    lambda h: host_W[h])
    for t in range(T):
        want = full[t].copy()
        for i in range(k):
            if idx[t, i] == e and slot[t, i] < 0:
                want -= w[t, i] * oracle.expert_ffn(x[t:t + 1], *W[e])[0]
        np.testing.assert_allclose(got[t], want, rtol=1e-9, atol=1e-12)


def test_verify_equals_separate_tokens():
    E, d, f, k = 10, 64, 32, 3
    W, Wsh = _tiny_layer(E, d, f)
    allW = W + [Wsh]
    rng = np.random.default_rng(2)
    x = rng.normal(size=(4, d))
    logits = rng.normal(size=(4, E)).astype(np.float32)
    idx, w = oracle.route_topk(logits, k)
    y4 = oracle.layer_decode(x, idx, idx, w, lambda s: allW[s], E)
    for t in range(4):
        y1 = oracle.layer_decode(x[t:t + 1], idx[t:t + 1], idx[t:t + 1], w[t:t + 1],
                                 lambda s: allW[s], E)
        np.testing.assert_array_equal(y4[t], y1[0])
    plan = oracle.union_plan(idx, idx, E)
    seen = [s for s, _ in plan]
    assert len(seen) == len(set(seen)) and seen[-1] == E
    assert set(seen[:-1]) == set(idx.reshape(-1).tolist())
    for s, toks in plan[:-1]:
        assert toks == [t for t in range(4) if s in idx[t]]


def test_combine_linear_and_selects():
    rng = np.random.default_rng(4)
    T, k, d, R = 5, 3, 16, 15
    x = rng.normal(size=(T, d))
    A = rng.normal(size=(R, d))
    B = rng.normal(size=(R, d))
    pos = rng.permutation(R).reshape(T, k).astype(np.int32)
    pos[1, 2] = -1
    w = rng.random((T, k))
    sh = rng.normal(size=(T, d))
    ya = oracle.combine(x, A, pos, w, sh) - x - sh
    yb = oracle.combine(x, B, pos, w, sh) - x - sh
    yab = oracle.combine(x, 2.0 * A - 3.0 * B, pos, w, sh) - x - sh
    np.testing.assert_allclose(yab, 2.0 * ya - 3.0 * yb, rtol=1e-12, atol=1e-12)
    onehot = np.zeros((T, k))
    onehot[:, 1] = 1.0
    y = oracle.combine(x, A, pos, onehot)
    np.testing.assert_allclose(y, x + A[pos[:, 1]], rtol=0, atol=1e-15)
    y = oracle.combine(x, A, pos, w)
    assert np.allclose(y[1], x[1] + w[1, 0] * A[pos[1, 0]] + w[1, 1] * A[pos[1, 1]])
