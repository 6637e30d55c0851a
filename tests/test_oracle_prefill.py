"""Pins of the oracle's prefill chunk (CPU).

* bf16_round equals torch's float32 -> bfloat16 conversion (round to nearest
  even) on fp32-representable values, including exact ties and subnormals
* permute_pairs: perm is a bijection, offsets are the prefix sums of the
  group sizes, order inside a group is by (t, i), pair_pos inverts perm
* prefill_layer equals a per-token loop over expert_ffn_bf16 (checks the
  permutation and un-permutation) and stays within the bf16 rounding bound
  of the unrounded layer
"""
import numpy as np
import torch

import oracle
import synth


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.normal(size=20000).astype(np.float32),
        (rng.normal(size=2000) * 1e-38).astype(np.float32),       # subnormal range
        (rng.normal(size=2000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0], np.float32),
    ])
    # exact ties: bf16 value plus half an ulp (both even and odd last bits)
    base = torch.tensor(rng.normal(size=500).astype(np.float32)).to(torch.bfloat16).float().numpy()
    ties = (base.view(np.uint32) + np.uint32(0x8000)).view(np.float32)
    v = np.concatenate([v, ties])
    ref = torch.tensor(v).to(torch.bfloat16).double().numpy()
    got = oracle.bf16_round(v.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_permute_invariants():
    rng = np.random.default_rng(1)
    T, E, k = 50, 12, 4
    logits = rng.normal(size=(T, E)).astype(np.float32)
    idx, _ = oracle.route_topk(logits, k)
    off, perm, pos = oracle.permute_pairs(idx, E)
    assert sorted(perm.tolist()) == list(range(T * k))
    counts = np.bincount(idx.reshape(-1), minlength=E)
    np.testing.assert_array_equal(np.diff(off), counts)
    assert off[0] == 0 and off[-1] == T * k
    for e in range(E):
        seg = perm[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(idx.reshape(-1)[seg] == e)
    np.testing.assert_array_equal(pos.reshape(-1)[perm], np.arange(T * k))


def test_prefill_matches_per_token_definition():
    E, d, f, k, T = 6, 64, 32, 3, 16
    gen = torch.Generator().manual_seed(11)
    G = torch.randn(E + 1, 2 * f, d, generator=gen) * 0.05
    D = torch.randn(E + 1, d, f, generator=gen) * 0.05
    slots = synth.pack_expert_slots(G, D, synth.FMT_Q2SM).numpy()
    W = [oracle.unpack_expert(s, oracle.FMT_Q2SM, d, f) for s in slots]
    rng = np.random.default_rng(3)
    x = torch.tensor(rng.normal(size=(T, d)), dtype=torch.float32).to(torch.bfloat16).double().numpy()
    logits = rng.normal(0, 1.5, size=(T, E)).astype(np.float32)
    idx, w = oracle.route_topk(logits, k)
    out_pairs, out_sh, y = oracle.prefill_layer(x, idx, w, lambda e: W[e], W[E], E)
    ref = x.copy()
    for t in range(T):
        for i in range(k):
            ref[t] += w[t, i] * oracle.expert_ffn_bf16(x[t:t + 1], *W[idx[t, i]])[0]
        ref[t] += oracle.expert_ffn_bf16(x[t:t + 1], *W[E])[0]
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-14)
    # the rounding points move the result only by about bf16 precision
    y64 = oracle.layer_decode(x, idx, idx, w, lambda s: W[s], E)
    delta = np.abs(y64 - x).max()
    assert np.abs(y - y64).max() <= 2.0 ** -6 * delta
