"""GPU parity: the decode layer with its combine accumulated into buffers
(moe_decode_layer_acc, moe_decode_acc_finish).

The routing outputs must equal moe_decode_layer's bit for bit; the buffers
to clear must be zero; the previous layer's y formed as a side job must equal
x + the 8 buffers added in order (bit for bit, against torch's own adds in that
order); and x + the 8 accumulated buffers must match the oracle's layer within
the fp32 bounds (the order of the atomic additions varies, so the comparison
with moe_decode_layer's y is within the same bounds, not bitwise).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import GpuLayer, check_close, need_gpu

pytestmark = pytest.mark.gpu

NB = 8


def _in_order(x, acc):
    s = x.clone()
    for b in range(NB):
        s = s + acc[b]
    return s


def _check_layer(L, x, logits):
    import bit_expert_ffn_top_amd as bf
    dev = x.device
    T, d = x.shape
    k = L.shape.top_k
    tab = L.table_dev(dev)
    ref = bf.decode_layer(L.layer_obj, x, logits, tab)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    acc = torch.zeros((NB, T, d), device=dev)
    clear = torch.full((NB, T, d), 7.0, device=dev)
    prev_x = torch.randn((T, d), device=dev, generator=g)
    prev_acc = torch.randn((NB, T, d), device=dev, generator=g)
    prev_y = torch.full((T, d), float("nan"), device=dev)
    got = bf.decode_layer_acc(L.layer_obj, x, logits, tab, acc, acc_clear=clear,
                              prev=(prev_x, prev_acc, prev_y))
    y = bf.decode_acc_finish(x, acc)
    torch.cuda.synchronize()
    ry, ridx, rw, rslot, rme, rmp, rnm = [t.cpu() for t in ref]
    idx, w, slot, me, mp, nm = [t.cpu() for t in got]
    assert torch.equal(idx, ridx)
    assert torch.equal(w, rw)
    assert torch.equal(slot, rslot)
    assert torch.equal(nm[:2], rnm[:2])
    assert torch.equal(me[:int(nm[0])], rme[:int(rnm[0])])
    assert torch.equal(mp[:int(nm[1])], rmp[:int(rnm[1])])
    assert not clear.any()
    assert torch.equal(prev_y, _in_order(prev_x, prev_acc))
    y = y.cpu().numpy()
    check_close(y, ry.numpy(), x.cpu().numpy())
    oidx, ow = oracle.route_topk(logits.cpu().numpy(), k)
    oslot, _, _, _ = oracle.cache_lookup(oidx, L.table)
    oy = oracle.layer_decode(x.cpu().double().numpy(), oidx, oslot, ow, L.weights_of_slot,
                             L.shared_slot if L.shared_slot >= 0 else None)
    check_close(y, oy, x.cpu().numpy())


CASES = [
    # name, shape, fmt, T, shared
    ("e64_q2s", synth.LayerShape(64, 4, 256, 128, False), synth.FMT_Q2S, 1, False),
    ("e100_q2sm_T3", synth.LayerShape(100, 5, 256, 128, True), synth.FMT_Q2SM, 3, True),
    ("e1024_q3g_T4_k16", synth.LayerShape(1024, 16, 128, 64, True), synth.FMT_Q3G, 4, True),
    ("e40_k1_T4", synth.LayerShape(40, 1, 512, 64, False), synth.FMT_Q2SM, 4, False),
    ("e1000_k64", synth.LayerShape(1000, 64, 64, 32, True), synth.FMT_Q2S, 1, True),
]


@pytest.mark.parametrize("name,shape,fmt,T,shared", CASES, ids=[c[0] for c in CASES])
def test_decode_acc_small(name, shape, fmt, T, shared):
    dev = need_gpu()
    L = GpuLayer(0, 5, shape, fmt, dev, shared=shared)
    x = synth.make_x(0, 5, T, shape.d_model).to(dev)
    logits = synth.make_logits(0, 5, T, shape.n_experts, 1.0).to(dev)
    _check_layer(L, x, logits)


@pytest.mark.parametrize("fmt,T", [(synth.FMT_Q2SM, 1), (synth.FMT_Q2SM, 4), (synth.FMT_Q3G, 4)])
def test_decode_acc_full_size(fmt, T):
    """E=512, top-10 + shared, d=2048, d_ff=768 (only the chosen experts'
    slots are filled)."""
    dev = need_gpu()
    shape = synth.config_shape(1)
    x = synth.make_x(1, 2, T, shape.d_model)
    logits = synth.make_logits(1, 2, T, shape.n_experts, 1.5)
    ridx, _ = oracle.route_topk(logits.numpy(), shape.top_k)
    L = GpuLayer(1, 2, shape, fmt, dev, only_experts=set(ridx.reshape(-1).tolist()))
    _check_layer(L, x.to(dev), logits.to(dev))


def test_decode_acc_chain_graph():
    """Four layers as a step: layer l adds into buffer l % 3, clears buffer
    (l+1) % 3 and forms layer l-1's y; a finish call forms the last y.  Each
    layer's y is within the fp32 bounds of moe_decode_layer's, eagerly and in
    three replays of the captured step with other work in between."""
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    shape = synth.LayerShape(128, 6, 512, 256, True)
    T, d, n_layers = 2, shape.d_model, 4
    layers = [GpuLayer(2, l, shape, synth.FMT_Q2SM, dev) for l in range(n_layers)]
    xs = [synth.make_x(2, l, T, d).to(dev) for l in range(n_layers)]
    lgs = [synth.make_logits(2, l, T, shape.n_experts, 1.5).to(dev) for l in range(n_layers)]
    tabs = [L.table_dev(dev) for L in layers]
    refs = [bf.decode_layer(L.layer_obj, xs[l], lgs[l], tabs[l])[0].cpu()
            for l, L in enumerate(layers)]
    acc = [torch.zeros((NB, T, d), device=dev) for _ in range(3)]
    ys = [torch.empty((T, d), device=dev) for _ in range(n_layers)]

    def step():
        for l, L in enumerate(layers):
            prev = (xs[l - 1], acc[(l - 1) % 3], ys[l - 1]) if l else None
            bf.decode_layer_acc(L.layer_obj, xs[l], lgs[l], tabs[l], acc[l % 3],
                                acc_clear=acc[(l + 1) % 3], prev=prev)
        bf.decode_acc_finish(xs[-1], acc[(n_layers - 1) % 3], y=ys[-1])

    def check():
        torch.cuda.synchronize()
        for l in range(n_layers):
            check_close(ys[l].cpu().numpy(), refs[l].numpy(), xs[l].cpu().numpy())

    # the step's first layer adds into buffer 0: zero it before each step
    acc[0].zero_()
    step()
    check()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        acc[0].zero_()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step()
    torch.cuda.synchronize()
    for r in range(3):
        acc[0].zero_()          # outside the graph (no memset node in it)
        for y in ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        check()
        _ = (xs[0] * 2.0).sum().item()   # other work between replays
