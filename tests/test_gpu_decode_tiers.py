"""GPU parity: the two-tier decode layer in one launch (moe_decode_layer_tiers).

The resident chosen experts are read from the GPU pool and the missed ones
from the host tier in the same kernel, and all terms are joined in one sum.
The output must equal the oracle's two-tier layer within the fp32 bounds for
every rank limit; the routing outputs must be those of moe_decode_layer bit
for bit; with nothing missed y must be moe_decode_layer's y bit for bit; two
calls and graph replays must give the same bits; slots outside either pool
must count as absent.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import GpuLayer, HostTier, check_close, need_gpu

pytestmark = pytest.mark.gpu


def _tiers(L, H, x, logits, max_rank=None, host_table=None):
    import bit_expert_ffn_top_amd as bf
    htab = H.table_dev() if host_table is None else host_table
    out = bf.decode_layer_tiers(L.layer_obj, H.tier, x, logits, L.table_dev(x.device), htab,
                                max_rank=max_rank)
    torch.cuda.synchronize()
    return out


def _oracle(L, H, x, idx, w, slot, max_rank, host_slot=None):
    return oracle.layer_decode_tiers(
        x.cpu().double().numpy(), idx, w.astype(np.float64), slot, L.weights_of_slot,
        L.shared_slot if L.shared_slot >= 0 else None,
        H.host_slot if host_slot is None else host_slot, H.weights_of_host_slot, max_rank)


def _same_routing(a, b):
    """Routing outputs of two layer calls: idx, w, slot, the miss lists and
    their counts, bit for bit."""
    _, idx, w, slot, me, mp, nm = a
    _, idx2, w2, slot2, me2, mp2, nm2 = b
    assert torch.equal(idx, idx2) and torch.equal(slot, slot2)
    assert torch.equal(w.view(torch.int32), w2.view(torch.int32))
    assert torch.equal(nm[:2], nm2[:2])
    nd, npairs = int(nm[0]), int(nm[1])
    assert torch.equal(me[:nd], me2[:nd]) and torch.equal(mp[:npairs], mp2[:npairs])


def _chosen(logits, k):
    idx, _ = oracle.route_topk(logits.numpy(), k)
    return set(idx.reshape(-1).tolist())


@pytest.mark.parametrize("fmt,T,max_rank", [(synth.FMT_Q2SM, 1, None), (synth.FMT_Q2SM, 4, None),
                                            (synth.FMT_Q3G, 4, 5), (synth.FMT_Q2S, 2, 3)])
def test_tiers_full_size_zipf(fmt, T, max_rank):
    """E=512, top-10 + shared, d=2048, d_ff=768; 94 experts resident on the
    GPU (Zipf residency), the whole layer in pinned host memory."""
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    shape = synth.config_shape(2)
    c = synth.WORKLOADS[2]
    table, _, slot_expert = synth.make_slot_table(2, 1)
    resident = [e for e in slot_expert if e < shape.n_experts]
    x = synth.make_x(2, 1, T, shape.d_model)
    r = shape.top_k if max_rank is None else max_rank
    for step in range(100 * fmt + 7 * T, 100 * fmt + 7 * T + 100):
        logits = synth.zipf_gumbel_logits(2, 1, T, shape.n_experts, c["zipf_s"], step=step)
        ridx, _ = oracle.route_topk(logits.numpy(), shape.top_k)
        miss = table[ridx] < 0
        if (not miss.all() and miss[:, :r].any()
                and (r == shape.top_k or miss[:, r:].any())):
            break
    else:
        raise AssertionError("no routing of the wanted kind")
    chosen = _chosen(logits, shape.top_k)
    L = GpuLayer(2, 1, shape, fmt, dev, resident=resident, only_experts=chosen)
    H = HostTier(2, 1, shape, fmt, chosen)
    xd, ld = x.to(dev), logits.to(dev)
    out = _tiers(L, H, xd, ld, max_rank)
    y, idx, w, slot = (t.cpu() for t in out[:4])
    assert (slot < 0).any() and (slot >= 0).any()
    ref = _oracle(L, H, x, idx.numpy(), w.numpy(), slot.numpy(), max_rank)
    check_close(y.numpy(), ref, x.numpy())
    # routing and lookup exactly as the one-tier layer gives them
    single = bf.decode_layer(L.layer_obj, xd, ld, L.table_dev(dev))
    torch.cuda.synchronize()
    _same_routing(out, single)
    # the misses' part alone against the oracle
    part = _oracle(L, H, x, idx.numpy(), w.numpy(), slot.numpy(), 0)
    check_close((y - single[0].cpu()).numpy(), ref - part, what="misses")
    # a second call gives the same bits
    again = _tiers(L, H, xd, ld, max_rank)
    assert torch.equal(again[0].cpu(), y)


CASES = [
    # name, shape, fmt, T, shared, resident fraction, max ranks
    ("e100_k5_T3_q2s", synth.LayerShape(100, 5, 256, 128, True), synth.FMT_Q2S, 3, True, 0.5,
     (0, 1, 3, 5)),
    ("e300_k12_T4_q3g", synth.LayerShape(300, 12, 128, 64, False), synth.FMT_Q3G, 4, False, 0.3,
     (12, 7)),
    ("e1000_k16_T4_q2sm", synth.LayerShape(1000, 16, 64, 32, True), synth.FMT_Q2SM, 4, True, 0.1,
     (16, 2)),
    ("e64_k1_T1_q2sm", synth.LayerShape(64, 1, 512, 96, True), synth.FMT_Q2SM, 1, True, 0.0,
     (1, 0)),
    ("e64_k4_T1_q2s", synth.LayerShape(64, 4, 192, 160, False), synth.FMT_Q2S, 1, False, 0.25,
     (4, 2)),
]


@pytest.mark.parametrize("name,shape,fmt,T,shared,frac,ranks", CASES, ids=[c[0] for c in CASES])
def test_tiers_small(name, shape, fmt, T, shared, frac, ranks):
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    E = shape.n_experts
    rng = np.random.default_rng(len(name) + 17)
    resident = sorted(rng.choice(E, int(frac * E), replace=False).tolist())
    L = GpuLayer(0, 4, shape, fmt, dev, resident=resident, shared=shared)
    x = synth.make_x(0, 4, T, shape.d_model)
    logits = synth.make_logits(0, 4, T, E, 1.0)
    chosen = _chosen(logits, shape.top_k)
    missed = sorted(chosen - set(resident))
    absent = missed[:1] if len(missed) > 1 else []   # one missed expert in neither tier
    H = HostTier(0, 4, shape, fmt, chosen, absent=absent, seed=5)
    xd, ld = x.to(dev), logits.to(dev)
    single = bf.decode_layer(L.layer_obj, xd, ld, L.table_dev(dev))
    torch.cuda.synchronize()
    for r in ranks:
        out = _tiers(L, H, xd, ld, r)
        _same_routing(out, single)
        y, idx, w, slot = (t.cpu() for t in out[:4])
        ref = _oracle(L, H, x, idx.numpy(), w.numpy(), slot.numpy(), r)
        check_close(y.numpy(), ref, x.numpy())
        if r == 0:   # no miss runs: the one-tier layer's sum, so its bits
            assert torch.equal(out[0], single[0])


def test_tiers_host_slots_outside_the_pool_are_absent():
    """Host slots at or past H->n_slots, or negative other than -1, add
    nothing (like -1); the resident part is unaffected."""
    dev = need_gpu()
    shape = synth.LayerShape(128, 8, 256, 128, True)
    T = 4
    rng = np.random.default_rng(31)
    resident = sorted(rng.choice(128, 40, replace=False).tolist())
    L = GpuLayer(0, 6, shape, synth.FMT_Q2SM, dev, resident=resident)
    x = synth.make_x(0, 6, T, shape.d_model)
    logits = synth.make_logits(0, 6, T, 128, 1.0)
    chosen = _chosen(logits, 8)
    H = HostTier(0, 6, shape, synth.FMT_Q2SM, chosen, seed=6)
    missed = sorted(chosen - set(resident))
    assert len(missed) >= 3
    bad = H.host_slot.copy()
    bad[missed[0]] = 128                      # one past the last host slot
    bad[missed[1]] = 1 << 30
    bad[missed[2]] = -7
    xd, ld = x.to(dev), logits.to(dev)
    out = _tiers(L, H, xd, ld, None, host_table=torch.tensor(bad, device=dev))
    y, idx, w, slot = (t.cpu() for t in out[:4])
    seen = bad.copy()
    seen[missed[:3]] = -1
    ref = _oracle(L, H, x, idx.numpy(), w.numpy(), slot.numpy(), None, host_slot=seen)
    check_close(y.numpy(), ref, x.numpy())


def test_tiers_all_hits_equal_the_one_tier_layer():
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    shape = synth.LayerShape(64, 8, 256, 128, True)
    L = GpuLayer(0, 9, shape, synth.FMT_Q2S, dev)
    x = synth.make_x(0, 9, 3, shape.d_model).to(dev)
    logits = synth.make_logits(0, 9, 3, shape.n_experts, 1.0).to(dev)
    H = HostTier(0, 9, shape, synth.FMT_Q2S, [], seed=3)
    out = _tiers(L, H, x, logits)
    single = bf.decode_layer(L.layer_obj, x, logits, L.table_dev(dev))
    torch.cuda.synchronize()
    assert (out[3] >= 0).all()
    _same_routing(out, single)
    assert torch.equal(out[0], single[0])


def test_tiers_device_pool_and_empty_cache():
    """Nothing resident on the GPU but the shared expert (every pair read
    from the second tier, here in device memory); the layer equals the dense
    layer of every expert."""
    dev = need_gpu()
    shape = synth.LayerShape(64, 6, 256, 128, True)
    T = 4
    L = GpuLayer(0, 8, shape, synth.FMT_Q2SM, dev, resident=[], shared=True)
    x = synth.make_x(0, 8, T, shape.d_model)
    logits = synth.make_logits(0, 8, T, shape.n_experts, 1.0)
    H = HostTier(0, 8, shape, synth.FMT_Q2SM, range(shape.n_experts), device_pool=True, seed=2)
    out = _tiers(L, H, x.to(dev), logits.to(dev))
    assert (out[3] < 0).all()
    expert_w = [H.weights_of_host_slot(int(H.host_slot[e])) for e in range(shape.n_experts)]
    ref = oracle.layer_dense_mixture(x.double().numpy(), logits.numpy(), expert_w, shape.top_k,
                                     L.weights_of_slot(L.shared_slot))
    check_close(out[0].cpu().numpy(), ref, x.numpy())


def test_tiers_close_to_the_two_call_layer():
    """The same terms as moe_decode_layer followed by moe_decode_misses (only
    the order of the fp32 additions differs)."""
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    shape = synth.LayerShape(200, 10, 512, 256, True)
    T = 2
    rng = np.random.default_rng(4)
    resident = sorted(rng.choice(200, 60, replace=False).tolist())
    L = GpuLayer(0, 10, shape, synth.FMT_Q2SM, dev, resident=resident)
    x = synth.make_x(0, 10, T, shape.d_model).to(dev)
    logits = synth.make_logits(0, 10, T, 200, 1.0)
    H = HostTier(0, 10, shape, synth.FMT_Q2SM, _chosen(logits, 10), seed=4)
    logits = logits.to(dev)
    out = _tiers(L, H, x, logits, 6)
    y2, idx, w, slot, _, _, _ = bf.decode_layer(L.layer_obj, x, logits, L.table_dev(dev))
    bf.decode_misses(H.tier, x, idx, slot, w, H.table_dev(), y2, max_rank=6)
    torch.cuda.synchronize()
    assert (slot < 0).any()
    check_close(out[0].cpu().numpy(), y2.cpu().double().numpy(), x.cpu().numpy(),
                what="tiers vs two calls")


def test_tiers_graph_replay_matches_eager():
    """The layer captured in a graph, replayed three times with eager work in
    between; every replay equals the eager result bit for bit."""
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    shape = synth.LayerShape(200, 10, 512, 256, True)
    T = 4
    rng = np.random.default_rng(8)
    resident = sorted(rng.choice(200, 50, replace=False).tolist())
    L = GpuLayer(0, 11, shape, synth.FMT_Q2SM, dev, resident=resident)
    x = synth.make_x(0, 11, T, shape.d_model).to(dev)
    logits = synth.make_logits(0, 11, T, 200, 1.0)
    H = HostTier(0, 11, shape, synth.FMT_Q2SM, _chosen(logits, 10), seed=7)
    logits = logits.to(dev)
    tab, htab = L.table_dev(dev), H.table_dev()
    k = shape.top_k
    bufs = dict(idx=torch.empty((T, k), dtype=torch.int32, device=dev),
                w=torch.empty((T, k), dtype=torch.float32, device=dev),
                slot=torch.empty((T, k), dtype=torch.int32, device=dev),
                miss_expert=torch.empty((T * k,), dtype=torch.int32, device=dev),
                miss_pair=torch.empty((T * k,), dtype=torch.int32, device=dev),
                n_miss=torch.empty((4,), dtype=torch.int32, device=dev),
                y=torch.empty((T, shape.d_model), dtype=torch.float32, device=dev))
    ws = torch.empty((bf.decode_workspace_bytes(L.layer_obj, T),), dtype=torch.uint8, device=dev)

    def step():
        bf.decode_layer_tiers(L.layer_obj, H.tier, x, logits, tab, htab, ws=ws, **bufs)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = bufs["y"].clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        bufs["y"].fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs["y"], eager)
        step()
        torch.cuda.synchronize()
    ref = _oracle(L, H, x, bufs["idx"].cpu().numpy(), bufs["w"].cpu().numpy(),
                  bufs["slot"].cpu().numpy(), None)
    check_close(eager.cpu().numpy(), ref, x.cpu().numpy())
