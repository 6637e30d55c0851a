"""GPU parity: expert-cache admission and eviction.

moe_cache_count, moe_cache_plan and moe_cache_commit must give exactly the
oracle's counts, tables and swap lists (integer work: bit for bit);
moe_cache_fill must copy exactly the planned slots' bytes and nothing else;
a run of decode steps that adapts its cache must match the oracle's
simulation of the same policy step by step (tables bit for bit, y within the
fp32 bounds) and raise the hit rate when routing concentrates.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import GpuLayer, check_close, need_gpu

pytestmark = pytest.mark.gpu


def _dev_i32(a, dev):
    return torch.tensor(np.asarray(a).astype(np.int64).astype(np.int32), dtype=torch.int32,
                        device=dev)


def _u32(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("E,n", [(512, 40960), (1000, 64), (7, 1000)])
def test_count_matches_oracle(E, n):
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    rng = np.random.default_rng(E)
    idx = rng.integers(-3, E + 3, n).astype(np.int32)         # a few ids out of range
    c0 = rng.integers(0, 2**32, E, dtype=np.uint64).astype(np.uint32)
    c0[:2] = 0xFFFFFFFF                                        # wraps
    counts = torch.tensor(c0.view(np.int32), device=dev)
    bf.cache_count(_dev_i32(idx, dev), counts)
    torch.cuda.synchronize()
    ok = idx[(idx >= 0) & (idx < E)]
    np.testing.assert_array_equal(_u32(counts), oracle.cache_count(c0, ok))


def _random_state(rng, E, n_slots, shared_slot, n_res, n_missing, count_hi):
    eos = np.full(n_slots, -1, np.int32)
    slots = [s for s in range(n_slots) if s != shared_slot]
    rng.shuffle(slots)
    res = rng.choice(E, min(n_res, len(slots), E), replace=False)
    for s, e in zip(slots, res):
        eos[s] = e
    if shared_slot >= 0:
        eos[shared_slot] = E
    soe = np.full(E, -1, np.int32)
    for s, e in enumerate(eos):
        if 0 <= e < E:
            soe[e] = s
    hs = rng.permutation(E).astype(np.int32)
    hs[rng.choice(E, n_missing, replace=False)] = -1
    cnt = rng.integers(0, count_hi, E).astype(np.uint32)
    return cnt, soe, eos, hs


PLAN_CASES = [
    # E, n_slots, shared_slot, residents, host-missing, count range, max_swaps, shift
    (512, 95, 94, 94, 0, 40, 8, 1),
    (512, 95, 3, 60, 5, 3, 1024, 0),          # heavy ties, empty slots
    (1024, 4096, -1, 1000, 10, 100, 1024, 2),  # more slots than experts
    (64, 17, 16, 16, 0, 2, 5, 31),
    (300, 1, -1, 1, 0, 10, 3, 1),
    (40, 50, 49, 0, 39, 5, 64, 0),            # one expert with a host copy
]


@pytest.mark.parametrize("case", PLAN_CASES, ids=[f"E{c[0]}_s{c[1]}_m{c[6]}" for c in PLAN_CASES])
def test_plan_and_commit_match_oracle(case):
    import bit_expert_ffn_top_amd as bf
    E, n_slots, shared_slot, n_res, n_missing, hi, max_swaps, shift = case
    dev = need_gpu()
    rng = np.random.default_rng(n_slots + E)
    cnt, soe, eos, hs = _random_state(rng, E, n_slots, shared_slot, n_res, n_missing, hi)
    d_cnt = torch.tensor(cnt.view(np.int32), device=dev)
    d_soe, d_eos, d_hs = _dev_i32(soe, dev), _dev_i32(eos, dev), _dev_i32(hs, dev)
    swaps, n_sw = bf.cache_plan(d_cnt, d_soe, d_eos, shared_slot, d_hs, E, max_swaps, shift)
    torch.cuda.synchronize()
    r_cnt, r_soe, r_eos, r_sw = oracle.cache_plan(cnt, soe, eos, shared_slot, hs, E, max_swaps,
                                                  shift)
    n = int(n_sw[0])
    assert n == len(r_sw)
    np.testing.assert_array_equal(_u32(d_cnt), r_cnt)
    np.testing.assert_array_equal(d_soe.cpu().numpy(), r_soe)
    np.testing.assert_array_equal(d_eos.cpu().numpy(), r_eos)
    got = [tuple(int(v) for v in row) for row in swaps[:n].cpu().numpy()]
    assert got == r_sw
    bf.cache_commit(d_soe, swaps, n_sw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d_soe.cpu().numpy(), oracle.cache_commit(r_soe, r_sw))


def test_fill_copies_exactly_the_planned_slots():
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    shape = synth.LayerShape(96, 4, 256, 128, False)
    fmt = synth.FMT_Q3G
    sb = synth.slot_bytes(fmt, shape.d_model, shape.d_ff)
    E, n_slots = shape.n_experts, 20
    g = torch.Generator().manual_seed(3)
    host = torch.randint(0, 256, (E, sb), dtype=torch.uint8, generator=g).pin_memory()
    pool0 = torch.randint(0, 256, (n_slots, sb), dtype=torch.uint8, generator=g)
    pool = pool0.to(dev)
    L = bf.MoeLayer(shape.d_model, shape.d_ff, E, shape.top_k, fmt, pool, -1)
    H = bf.HostTier(shape.d_model, shape.d_ff, E, shape.top_k, fmt, host)
    rows = [(3, 7, 11, 50), (0, -1, 12, 95), (19, 2, 13, 0), (5, 1, 14, 200), (6, 1, 15, 1)]
    swaps = torch.full((8, 4), -1, dtype=torch.int32)
    swaps[:len(rows)] = torch.tensor(rows, dtype=torch.int32)
    n_sw = torch.tensor([4, 0, 0, 0], dtype=torch.int32)    # the fifth row is past the count
    bf.cache_fill(L, H, swaps.to(dev), n_sw.to(dev))
    torch.cuda.synchronize()
    want = pool0.clone()
    for s, _, _, h in rows[:4]:
        if h < E:                                           # host slot 200 is outside the tier
            want[s] = host[h]
    assert torch.equal(pool.cpu(), want)


def test_adaptive_cache_follows_routing():
    """Decode steps whose routing concentrates on a few experts that start
    out of the cache: count after every step, plan + fill + commit every
    third step; tables, swaps and y follow the oracle's simulation."""
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    shape = synth.LayerShape(48, 4, 256, 128, True)
    fmt = synth.FMT_Q2SM
    E, k, T = shape.n_experts, shape.top_k, 2
    n_slots = 13                                            # 12 cached experts + shared
    shared_slot = 12
    sb = synth.slot_bytes(fmt, shape.d_model, shape.d_ff)
    experts = list(range(E))
    host_packed = synth.make_layer_pool(0, 11, experts + [E], device=dev, fmt=fmt, shape=shape)
    host = host_packed[:E].cpu().pin_memory()
    hs = np.arange(E, dtype=np.int32)
    W = [oracle.unpack_expert(host_packed[e].cpu().numpy(), fmt, shape.d_model, shape.d_ff)
         for e in range(E + 1)]
    # initial cache: experts 0..11 in slots 0..11, shared expert in slot 12
    eos = np.array(list(range(12)) + [E], np.int32)
    soe = np.full(E, -1, np.int32)
    soe[:12] = np.arange(12)
    pool = torch.zeros((n_slots, sb), dtype=torch.uint8, device=dev)
    pool[:12] = host_packed[:12]
    pool[12] = host_packed[E]
    L = bf.MoeLayer(shape.d_model, shape.d_ff, E, k, fmt, pool, shared_slot)
    H = bf.HostTier(shape.d_model, shape.d_ff, E, k, fmt, host)
    d_soe, d_eos, d_hs = _dev_i32(soe, dev), _dev_i32(eos, dev), _dev_i32(hs, dev)
    d_cnt = torch.zeros(E, dtype=torch.int32, device=dev)
    cnt = np.zeros(E, np.uint32)
    rng = np.random.default_rng(5)
    favour = np.arange(30, 42)                              # popular later, not cached at first
    hits = []
    for step in range(12):
        x = torch.tensor(rng.normal(size=(T, shape.d_model)), dtype=torch.float32)
        lg = rng.normal(size=(T, E)).astype(np.float32)
        lg[:, favour] += 4.0
        y, idx, w, slot, _, _, _ = bf.decode_layer(L, x.to(dev), torch.tensor(lg).to(dev), d_soe)
        bf.decode_misses(H, x.to(dev), idx, slot, w, d_hs, y)
        bf.cache_count(idx, d_cnt)
        torch.cuda.synchronize()
        # oracle: the same step with its own copy of the policy state
        oidx, ow = oracle.route_topk(lg, k)
        oslot = soe[oidx]
        np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
        np.testing.assert_array_equal(slot.cpu().numpy(), oslot)
        ref = oracle.layer_decode_tiers(x.double().numpy(), oidx, ow, oslot,
                                        lambda s: W[int(eos[s])], shared_slot, hs,
                                        lambda h: W[h])
        check_close(y.cpu().numpy(), ref, x.numpy())
        hits.append(float((oslot >= 0).mean()))
        cnt = oracle.cache_count(cnt, oidx)
        if step % 3 == 2:
            swaps, n_sw = bf.cache_plan(d_cnt, d_soe, d_eos, shared_slot, d_hs, E, 4, 1)
            bf.cache_fill(L, H, swaps, n_sw)
            bf.cache_commit(d_soe, swaps, n_sw)
            torch.cuda.synchronize()
            cnt, soe, eos, r_sw = oracle.cache_plan(cnt, soe, eos, shared_slot, hs, E, 4, 1)
            soe = oracle.cache_commit(soe, r_sw)
            n = int(n_sw[0])
            assert [tuple(int(v) for v in r) for r in swaps[:n].cpu().numpy()] == r_sw
            np.testing.assert_array_equal(d_soe.cpu().numpy(), soe)
            np.testing.assert_array_equal(d_eos.cpu().numpy(), eos)
            np.testing.assert_array_equal(_u32(d_cnt), cnt)
            pc = pool.cpu()
            for s in range(12):
                assert torch.equal(pc[s], host_packed[int(eos[s])].cpu())
    assert np.mean(hits[-3:]) > np.mean(hits[:3]) + 0.3
