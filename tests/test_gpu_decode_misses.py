"""GPU parity: miss execution from the host tier and the per-layer join.

The GPU part (moe_decode_layer over the resident experts) followed by
moe_decode_misses (the missed experts read from a pinned host copy of the
layer) must equal the oracle's two-tier layer within the fp32 bounds, for
every rank limit; a step without misses must leave y bit for bit as it was;
graph replays must equal the eager call bit for bit; the two phases on two
streams (host-tier read overlapping the GPU part, join after both) must give
the serial call's bits; the host-side argument checks must refuse what the
header rules out.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import GpuLayer, HostTier, check_close, need_gpu

pytestmark = pytest.mark.gpu


def _run(L, H, x, logits, max_rank=None):
    import bit_expert_ffn_top_amd as bf
    dev = x.device
    y, idx, w, slot, _, _, nm = bf.decode_layer(L.layer_obj, x, logits, L.table_dev(dev))
    y_gpu = y.clone()
    bf.decode_misses(H.tier, x, idx, slot, w, H.table_dev(), y, max_rank=max_rank)
    torch.cuda.synchronize()
    return y.cpu(), y_gpu.cpu(), idx.cpu().numpy(), w.cpu().numpy(), slot.cpu().numpy()


def _oracle(L, H, x, idx, w, slot, max_rank):
    return oracle.layer_decode_tiers(
        x.cpu().double().numpy(), idx, w.astype(np.float64), slot, L.weights_of_slot,
        L.shared_slot if L.shared_slot >= 0 else None, H.host_slot, H.weights_of_host_slot,
        max_rank)


def _chosen(logits, k):
    idx, _ = oracle.route_topk(logits.numpy(), k)
    return set(idx.reshape(-1).tolist())


@pytest.mark.parametrize("fmt,T,max_rank", [(synth.FMT_Q2SM, 4, None), (synth.FMT_Q3G, 1, 5),
                                            (synth.FMT_Q2S, 2, 3)])
def test_misses_full_size_zipf(fmt, T, max_rank):
    """E=512, top-10 + shared, d=2048, d_ff=768; 94 experts resident on the
    GPU (Zipf residency), the whole layer in pinned host memory."""
    dev = need_gpu()
    shape = synth.config_shape(2)
    c = synth.WORKLOADS[2]
    _, _, slot_expert = synth.make_slot_table(2, 1)
    resident = [e for e in slot_expert if e < shape.n_experts]
    x = synth.make_x(2, 1, T, shape.d_model)
    table, _, _ = synth.make_slot_table(2, 1)
    r = shape.top_k if max_rank is None else max_rank
    for step in range(100 * fmt, 100 * fmt + 100):
        # first routing with hits, misses that run and (with a rank limit)
        # misses that are left out
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
    y, y_gpu, idx, w, slot = _run(L, H, x.to(dev), logits.to(dev), max_rank)
    assert (slot < 0).any() and (slot >= 0).any()
    ref = _oracle(L, H, x, idx, w, slot, max_rank)
    check_close(y.numpy(), ref, x.numpy())
    # the misses' contribution alone
    part = _oracle(L, H, x, idx, w, slot, 0)
    check_close((y - y_gpu).numpy(), ref - part, what="misses")


CASES = [
    # name, shape, fmt, T, shared, resident fraction, max ranks
    ("e100_k5_T3_q2s", synth.LayerShape(100, 5, 256, 128, True), synth.FMT_Q2S, 3, True, 0.5,
     (0, 1, 3, 5)),
    ("e300_k12_T4_q3g", synth.LayerShape(300, 12, 128, 64, False), synth.FMT_Q3G, 4, False, 0.3,
     (12, 7)),
    ("e1000_k16_T4_q2sm", synth.LayerShape(1000, 16, 64, 32, True), synth.FMT_Q2SM, 4, True, 0.1,
     (16,)),
]


@pytest.mark.parametrize("name,shape,fmt,T,shared,frac,ranks", CASES, ids=[c[0] for c in CASES])
def test_misses_small(name, shape, fmt, T, shared, frac, ranks):
    dev = need_gpu()
    E = shape.n_experts
    rng = np.random.default_rng(len(name))
    resident = sorted(rng.choice(E, int(frac * E), replace=False).tolist())
    L = GpuLayer(0, 3, shape, fmt, dev, resident=resident, shared=shared)
    x = synth.make_x(0, 3, T, shape.d_model)
    logits = synth.make_logits(0, 3, T, E, 1.0)
    chosen = _chosen(logits, shape.top_k)
    missed = sorted(chosen - set(resident))
    absent = missed[:1]                         # one missed expert in neither tier
    H = HostTier(0, 3, shape, fmt, chosen, absent=absent, seed=1)
    for r in ranks:
        y, y_gpu, idx, w, slot = _run(L, H, x.to(dev), logits.to(dev), r)
        ref = _oracle(L, H, x, idx, w, slot, r)
        check_close(y.numpy(), ref, x.numpy())
        if r == 0:
            assert torch.equal(y, y_gpu)


def test_misses_device_pool_and_empty_cache():
    """Nothing resident on the GPU but the shared expert (every pair a
    miss), the second tier in device memory; the joined layer equals the
    dense layer of every expert."""
    dev = need_gpu()
    shape = synth.LayerShape(64, 6, 256, 128, True)
    T = 4
    L = GpuLayer(0, 8, shape, synth.FMT_Q2SM, dev, resident=[], shared=True)
    x = synth.make_x(0, 8, T, shape.d_model)
    logits = synth.make_logits(0, 8, T, shape.n_experts, 1.0)
    H = HostTier(0, 8, shape, synth.FMT_Q2SM, range(shape.n_experts), device_pool=True, seed=2)
    y, _, idx, w, slot = _run(L, H, x.to(dev), logits.to(dev))
    assert (slot < 0).all()
    expert_w = [H.weights_of_host_slot(int(H.host_slot[e])) for e in range(shape.n_experts)]
    ref = oracle.layer_dense_mixture(x.double().numpy(), logits.numpy(), expert_w, shape.top_k,
                                     L.weights_of_slot(L.shared_slot))
    check_close(y.numpy(), ref, x.numpy())


def test_misses_all_hits_leave_y():
    dev = need_gpu()
    shape = synth.LayerShape(64, 8, 256, 128, True)
    L = GpuLayer(0, 9, shape, synth.FMT_Q2S, dev)
    x = synth.make_x(0, 9, 3, shape.d_model)
    logits = synth.make_logits(0, 9, 3, shape.n_experts, 1.0)
    H = HostTier(0, 9, shape, synth.FMT_Q2S, [], seed=3)
    y, y_gpu, _, _, slot = _run(L, H, x.to(dev), logits.to(dev))
    assert (slot >= 0).all()
    assert torch.equal(y, y_gpu)


def test_misses_graph_replay_matches_eager():
    """GPU part + misses captured in one graph, replayed three times with
    eager work in between; every replay equals the eager result bit for bit."""
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
        bf.decode_layer(L.layer_obj, x, logits, tab, ws=ws, **bufs)
        bf.decode_misses(H.tier, x, bufs["idx"], bufs["slot"], bufs["w"], htab, bufs["y"], ws=ws)

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
        step()                                    # eager work between replays
        torch.cuda.synchronize()
    ref = _oracle(L, H, x, bufs["idx"].cpu().numpy(), bufs["w"].cpu().numpy(),
                  bufs["slot"].cpu().numpy(), None)
    check_close(eager.cpu().numpy(), ref, x.cpu().numpy())


def _overlapped_step(bf, L, H, x, logits, tab, htab, bufs, ws_gpu, ws_miss, side, max_rank=None):
    """Routing and lookup, then the host-tier read on stream `side` while the
    GPU part runs on the current stream; the join after both."""
    main = torch.cuda.current_stream()
    k = L.shape.top_k
    bf.route_topk(logits, k, idx=bufs["idx"], w=bufs["w"])
    bf.cache_lookup(bufs["idx"], tab, slot=bufs["slot"], miss_expert=bufs["miss_expert"],
                    n_miss=bufs["n_miss"])
    side.wait_stream(main)
    with torch.cuda.stream(side):
        bf.decode_misses(H.tier, x, bufs["idx"], bufs["slot"], None, htab, None,
                         max_rank=max_rank, ws=ws_miss, phases=bf.MISSES_READ)
    bf.expert_ffn_decode(L.layer_obj, x, bufs["idx"], bufs["slot"], bufs["w"], y=bufs["y"],
                         ws=ws_gpu)
    main.wait_stream(side)
    bf.decode_misses(H.tier, None, bufs["idx"], bufs["slot"], bufs["w"], htab, bufs["y"],
                     max_rank=max_rank, ws=ws_miss, phases=bf.MISSES_JOIN)


@pytest.mark.parametrize("max_rank", [None, 4])
def test_misses_two_phases_on_two_streams(max_rank):
    """The host-tier read on a second stream, overlapping the GPU part, and
    the join after both: the same bits as the GPU part followed by
    moe_decode_misses, eager and in every replay of a captured graph."""
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    shape = synth.LayerShape(200, 10, 512, 256, True)
    T = 3
    rng = np.random.default_rng(8)
    resident = sorted(rng.choice(200, 70, replace=False).tolist())
    L = GpuLayer(0, 11, shape, synth.FMT_Q2SM, dev, resident=resident)
    x = synth.make_x(0, 11, T, shape.d_model).to(dev)
    logits = synth.make_logits(0, 11, T, 200, 1.0)
    H = HostTier(0, 11, shape, synth.FMT_Q2SM, _chosen(logits, 10), seed=8)
    logits = logits.to(dev)
    tab, htab = L.table_dev(dev), H.table_dev()
    k = shape.top_k
    y_ser, *_ = _run(L, H, x, logits, max_rank)
    bufs = dict(idx=torch.empty((T, k), dtype=torch.int32, device=dev),
                w=torch.empty((T, k), dtype=torch.float32, device=dev),
                slot=torch.empty((T, k), dtype=torch.int32, device=dev),
                miss_expert=torch.empty((T * k,), dtype=torch.int32, device=dev),
                n_miss=torch.empty((4,), dtype=torch.int32, device=dev),
                y=torch.empty((T, shape.d_model), dtype=torch.float32, device=dev))
    nb = bf.decode_workspace_bytes(L.layer_obj, T)
    ws_gpu = torch.empty((nb,), dtype=torch.uint8, device=dev)
    ws_miss = torch.empty((nb,), dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream()
    step = lambda: _overlapped_step(bf, L, H, x, logits, tab, htab, bufs, ws_gpu, ws_miss, side,
                                    max_rank)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(bufs["y"].cpu(), y_ser)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        bufs["y"].fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs["y"].cpu(), y_ser)
        step()                                    # eager work between replays
        torch.cuda.synchronize()


def test_misses_argument_checks():
    import bit_expert_ffn_top_amd as bf
    from bit_expert_ffn_top_amd import _binding as b
    dev = need_gpu()
    shape = synth.LayerShape(64, 4, 256, 128, False)
    T, k, d = 1, 4, 256
    sb = synth.slot_bytes(synth.FMT_Q2S, d, 128)
    x = torch.zeros((T, d), device=dev)
    y = torch.zeros((T, d), device=dev)
    idx = torch.arange(k, dtype=torch.int32, device=dev).reshape(T, k)
    slot = torch.full((T, k), -1, dtype=torch.int32, device=dev)
    w = torch.zeros((T, k), device=dev)
    tab = torch.arange(64, dtype=torch.int32, device=dev)
    ws = torch.empty((1 << 20,), dtype=torch.uint8, device=dev)
    lib = b.lib()

    def call(pool_ptr, shared=-1, max_rank=k, n_slots=64):
        L = b.MoeLayerC(d, 128, 64, k, synth.FMT_Q2S, n_slots, shared, 0, sb, pool_ptr)
        return lib.moe_decode_misses(ctypes.byref(L), x.data_ptr(), T, idx.data_ptr(),
                                     slot.data_ptr(), w.data_ptr(), tab.data_ptr(), max_rank,
                                     y.data_ptr(), ws.data_ptr(), ws.numel(), None)

    pageable = np.zeros(64 * sb + 4096, dtype=np.uint8)
    addr = (pageable.ctypes.data + 255) & ~255
    # pageable host memory (max_rank 0: nothing would be enqueued even if accepted)
    assert call(addr, max_rank=0) == -1
    pinned = torch.zeros((64, sb), dtype=torch.uint8, pin_memory=True)
    assert call(pinned.data_ptr(), shared=0) == -1      # shared expert in the host tier
    assert call(pinned.data_ptr(), max_rank=k + 1) == -1
    assert call(pinned.data_ptr(), max_rank=-1) == -1
    assert call(pinned.data_ptr()) == 0                 # all-zero weights: y stays 0
    torch.cuda.synchronize()
    assert not y.any()
    with pytest.raises(ValueError):
        bf.HostTier(d, 128, 64, k, synth.FMT_Q2S, torch.zeros((64, sb), dtype=torch.uint8))
