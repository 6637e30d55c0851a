"""GPU parity: router top-k and expert-cache lookup against the oracle.
Indices, slots, miss lists and counts must match bit for bit; weights within
1e-6 relative."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import need_gpu

pytestmark = pytest.mark.gpu


def _topk_check(logits_cpu, k, dev):
    import bit_expert_ffn_top_amd as bf
    idx, w = bf.route_topk(logits_cpu.to(dev), k)
    torch.cuda.synchronize()
    ridx, rw = oracle.route_topk(logits_cpu.numpy(), k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    np.testing.assert_allclose(w.cpu().double().numpy(), rw, rtol=1e-6, atol=1e-7)
    return idx, w


@pytest.mark.parametrize("T,E,k,sigma", [
    (1, 64, 4, 1.0),        # tiny plumbing layer
    (1, 512, 10, 1.5),      # decode layer
    (4, 512, 10, 1.5),      # verify step
    (37, 100, 7, 2.0),      # E not a multiple of 64, ragged T
    (5, 1024, 64, 1.0),     # largest E and k
    (3, 64, 64, 1.0),       # k = E: full order
    (2, 1, 1, 1.0),         # one expert
])
def test_topk_random(T, E, k, sigma):
    dev = need_gpu()
    g = torch.Generator().manual_seed(T * 1000 + E + k)
    logits = torch.randn((T, E), generator=g) * sigma
    _topk_check(logits, k, dev)


def test_topk_ties_and_special_values():
    dev = need_gpu()
    g = torch.Generator().manual_seed(5)
    logits = torch.randint(-2, 3, (16, 128), generator=g).float()   # many ties
    logits[0, :] = 0.0
    logits[1, ::2] = -0.0
    logits[2, 5] = float("nan")
    logits[2, 6] = float("inf")
    logits[3, :] = float("nan")
    logits[4, :3] = float("inf")
    logits[5, :] = -float("inf")
    logits[6, 7] = -float("inf")
    _topk_check(logits, 10, dev)


def test_topk_prefill_size():
    dev = need_gpu()
    logits = synth.make_logits(4, 0, 8192, 512, 1.5)
    import bit_expert_ffn_top_amd as bf
    idx, w = bf.route_topk(logits.to(dev), 10)
    torch.cuda.synchronize()
    # every token: compare a sample in full, and the whole tensor by properties
    sample = np.random.default_rng(0).choice(8192, 64, replace=False)
    ridx, rw = oracle.route_topk(logits.numpy()[sample], 10)
    np.testing.assert_array_equal(idx.cpu().numpy()[sample], ridx)
    np.testing.assert_allclose(w.cpu().double().numpy()[sample], rw, rtol=1e-6, atol=1e-7)
    ref = np.argsort(-logits.numpy(), axis=1, kind="stable")[:, :10]
    np.testing.assert_array_equal(idx.cpu().numpy(), ref)
    np.testing.assert_allclose(w.sum(1).cpu().numpy(), 1.0, atol=2e-6)


def test_topk_empty():
    dev = need_gpu()
    import bit_expert_ffn_top_amd as bf
    idx, w = bf.route_topk(torch.zeros((0, 64), device=dev), 4)
    assert idx.shape == (0, 4)


def _lookup_check(idx_np, table_np, dev):
    import bit_expert_ffn_top_amd as bf
    idx = torch.tensor(idx_np, dtype=torch.int32, device=dev)
    table = torch.tensor(table_np, dtype=torch.int32, device=dev)
    slot, me, mp, n = bf.cache_lookup(idx, table)
    torch.cuda.synchronize()
    rslot, rme, rmp, rn = oracle.cache_lookup(idx_np, table_np)
    n = n.cpu().numpy()
    np.testing.assert_array_equal(slot.cpu().numpy(), rslot)
    np.testing.assert_array_equal(n[:2], rn)
    np.testing.assert_array_equal(me.cpu().numpy()[:n[0]], rme)
    np.testing.assert_array_equal(mp.cpu().numpy()[:n[1]], rmp)


@pytest.mark.parametrize("T,E,k,n_res", [(1, 512, 10, 94), (4, 512, 10, 94), (1, 64, 4, 64),
                                         (4, 512, 10, 0), (100, 256, 8, 40), (8192, 512, 10, 94),
                                         (3000, 1024, 16, 500)])
def test_lookup_random(T, E, k, n_res):
    dev = need_gpu()
    rng = np.random.default_rng(T + E + k + n_res)
    table = np.full(E, -1, np.int32)
    res = rng.choice(E, n_res, replace=False)
    table[res] = rng.permutation(n_res) + 3
    logits = rng.normal(size=(T, E)).astype(np.float32)
    idx = np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int32)
    _lookup_check(idx, table, dev)


def test_lookup_zipf_layer_hit_rate():
    """The expert-cache workload: ~72% of chosen experts resident."""
    dev = need_gpu()
    c = synth.WORKLOADS[2]
    hits = total = 0
    for layer in range(4):
        table, _, _ = synth.make_slot_table(2, layer)
        logits = synth.zipf_gumbel_logits(2, layer, 64, 512, c["zipf_s"])
        idx = np.argsort(-logits.numpy(), axis=1, kind="stable")[:, :10].astype(np.int32)
        _lookup_check(idx, table, dev)
        hits += int((table[idx] >= 0).sum())
        total += idx.size
    assert 0.66 < hits / total < 0.78
