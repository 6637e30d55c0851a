"""GPU parity: decode / verify through a stack of layers (moe_decode_stack).

Per layer the routing outputs must equal the oracle's (indices, slots and miss
lists exactly, weights to 1e-6) and y the oracle's layer output within the fp32
bar, each layer fed the input the kernel formed (x_l = y_{l-1} + addend_l,
recomputed here in fp32 from the returned y, so errors do not compound).
Bitwise properties: reruns, each token of a 4-token step against the same
token alone, many layers in one call against one layer per call, one layer
against moe_decode_layer, graph replays against the eager call.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import GpuLayer, check_close, need_gpu

pytestmark = pytest.mark.gpu


def _inputs(cfg, shape, T, nl, dev, sigma=1.5, step=0, addend_scale=0.5):
    x = synth.make_x(cfg, 0, T, shape.d_model, step=step).to(dev)
    logits = [synth.make_logits(cfg, 100 + l, T, shape.n_experts, sigma, step=step).to(dev)
              for l in range(nl)]
    adds = [addend_scale * synth.make_x(cfg, 200 + l, T, shape.d_model, step=step).to(dev)
            for l in range(nl)]
    return x, logits, adds


def _run(layers, x, logits, tables, adds, **kw):
    import bit_expert_ffn_top_amd as bf
    out = bf.decode_stack([L.layer_obj for L in layers], x, logits, tables, addends=adds,
                          routing=True, **kw)
    torch.cuda.synchronize()
    return out


def _check_against_oracle(layers, x, logits, adds, out, tables_host):
    k = layers[0].shape.top_k
    ys = out["y"].cpu()
    xl = x.cpu()
    for l, L in enumerate(layers):
        if l > 0:
            xl = ys[l - 1] + adds[l].cpu()          # fp32, as the kernel forms it
        lg = logits[l].cpu().numpy()
        oidx, ow = oracle.route_topk(lg, k)
        np.testing.assert_array_equal(out["idx"][l].cpu().numpy(), oidx)
        np.testing.assert_allclose(out["w"][l].cpu().numpy(), ow, rtol=1e-6, atol=0)
        oslot, ome, omp, onm = oracle.cache_lookup(oidx, tables_host[l])
        np.testing.assert_array_equal(out["slot"][l].cpu().numpy(), oslot)
        nm = out["n_miss"][l].cpu().numpy()
        assert list(nm[:2]) == list(onm)
        np.testing.assert_array_equal(out["miss_expert"][l].cpu().numpy()[:onm[0]], ome)
        np.testing.assert_array_equal(out["miss_pair"][l].cpu().numpy()[:onm[1]], omp)
        oy = oracle.layer_decode(xl.double().numpy(), oidx, oslot, ow, L.weights_of_slot,
                                 L.shared_slot if L.shared_slot >= 0 else None)
        check_close(ys[l].numpy(), oy, xl.numpy(), what=f"y[{l}]")


CASES = [
    # name, shape, T, formats per layer, resident fraction
    ("e64_k4_T1", synth.LayerShape(64, 4, 256, 128, False), 1,
     (synth.FMT_Q2S, synth.FMT_Q2SM, synth.FMT_Q3G), 1.0),
    ("e100_k5_T3_cache", synth.LayerShape(100, 5, 256, 128, True), 3,
     (synth.FMT_Q2SM, synth.FMT_Q3G, synth.FMT_Q2SM), 0.6),
    ("e1024_k16_T4", synth.LayerShape(1024, 16, 128, 64, True), 4,
     (synth.FMT_Q3G, synth.FMT_Q2SM), 1.0),
    ("e300_k12_T4_d2048", synth.LayerShape(300, 12, 2048, 96, True), 4,
     (synth.FMT_Q2SM, synth.FMT_Q2S), 0.8),
    ("e1000_k64_T1_d64", synth.LayerShape(1000, 64, 64, 32, True), 1,
     (synth.FMT_Q2S, synth.FMT_Q3G), 1.0),
    # 32 routed + shared = 33 members x 8 tiles = 264 tiles: the left-over
    # tiles are split one h index per workgroup on a 256-CU device
    ("e64_k32_T1_f256_split", synth.LayerShape(64, 32, 128, 256, True), 1,
     (synth.FMT_Q2SM, synth.FMT_Q3G, synth.FMT_Q2S), 1.0),
]


def _layers(cfg, shape, fmts, frac, dev, only=None):
    layers, tabs = [], []
    for l, fmt in enumerate(fmts):
        E = shape.n_experts
        rng = np.random.default_rng(77 + l)
        resident = np.arange(E) if frac >= 1.0 else np.sort(
            rng.choice(E, int(round(frac * E)), replace=False))
        L = GpuLayer(cfg, 300 + l, shape, fmt, dev, resident=resident, shared=shape.shared,
                     only_experts=None if only is None else only[l])
        layers.append(L)
        tabs.append(L.table)
    return layers, tabs


@pytest.mark.parametrize("name,shape,T,fmts,frac", CASES, ids=[c[0] for c in CASES])
def test_stack_small_vs_oracle(name, shape, T, fmts, frac):
    dev = need_gpu()
    layers, tabs = _layers(0, shape, fmts, frac, dev)
    x, logits, adds = _inputs(0, shape, T, len(fmts), dev, sigma=1.0)
    tables = [torch.tensor(t, dtype=torch.int32, device=dev) for t in tabs]
    out = _run(layers, x, logits, tables, adds)
    _check_against_oracle(layers, x, logits, adds, out, tabs)


@pytest.mark.parametrize("T,fmts", [(1, (synth.FMT_Q2SM, synth.FMT_Q3G, synth.FMT_Q2SM)),
                                    (3, (synth.FMT_Q2S, synth.FMT_Q2SM)),
                                    (4, (synth.FMT_Q2SM, synth.FMT_Q3G))])
def test_stack_full_size(T, fmts):
    """E=512, top-10 + shared, d=2048, d_ff=768, every expert resident under a
    seeded slot permutation (11 members x 24 tiles = 264 at T = 1); only the
    chosen experts' slots are filled."""
    dev = need_gpu()
    shape = synth.config_shape(1)
    nl = len(fmts)
    x, logits, adds = _inputs(1, shape, T, nl, dev, sigma=1.5)
    only = [set(oracle.route_topk(logits[l].cpu().numpy(), shape.top_k)[0].reshape(-1).tolist())
            for l in range(nl)]
    layers, tabs = _layers(1, shape, fmts, 1.0, dev, only=only)
    tables = [torch.tensor(t, dtype=torch.int32, device=dev) for t in tabs]
    out = _run(layers, x, logits, tables, adds)
    _check_against_oracle(layers, x, logits, adds, out, tabs)


def test_stack_bitwise_properties():
    """Reruns (a workspace reused, one filled with garbage) give the same
    bits; each token of a 4-token step has the bits it gets alone."""
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    shape = synth.LayerShape(200, 8, 512, 256, True)
    fmts = (synth.FMT_Q2SM, synth.FMT_Q3G, synth.FMT_Q2S, synth.FMT_Q2SM)
    layers, tabs = _layers(0, shape, fmts, 0.7, dev)
    tables = [torch.tensor(t, dtype=torch.int32, device=dev) for t in tabs]
    T = 4
    x, logits, adds = _inputs(0, shape, T, len(fmts), dev, sigma=1.0, step=3)
    a = _run(layers, x, logits, tables, adds)
    ws = a["ws"]
    b = _run(layers, x, logits, tables, adds, ws=ws)
    ws.fill_(0xA5)
    c = _run(layers, x, logits, tables, adds, ws=ws)
    for key in ("y", "idx", "w", "slot", "n_miss"):
        assert torch.equal(a[key], b[key]), key
        assert torch.equal(a[key], c[key]), key
    for t in range(T):
        s = _run(layers, x[t:t + 1].contiguous(), [lg[t:t + 1].contiguous() for lg in logits],
                 tables, [ad[t:t + 1].contiguous() for ad in adds])
        assert torch.equal(s["y"][:, 0], a["y"][:, t]), t
        assert torch.equal(s["idx"][:, 0], a["idx"][:, t]), t
        assert torch.equal(s["w"][:, 0], a["w"][:, t]), t
    _check_against_oracle(layers, x, logits, adds, a, tabs)


def test_stack_many_layers_equals_one_layer_calls():
    """18 layers in one call against 18 one-layer calls chained here with
    the same fp32 additions: the same bits."""
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    shape = synth.LayerShape(64, 4, 128, 64, True)
    nl = 18
    fmts = [(synth.FMT_Q2S, synth.FMT_Q2SM, synth.FMT_Q3G)[l % 3] for l in range(nl)]
    layers, tabs = _layers(0, shape, fmts, 0.75, dev)
    tables = [torch.tensor(t, dtype=torch.int32, device=dev) for t in tabs]
    T = 2
    x, logits, adds = _inputs(0, shape, T, nl, dev, sigma=1.0, step=5)
    full = _run(layers, x, logits, tables, adds)
    xl = x
    for l in range(nl):
        one = _run([layers[l]], xl, [logits[l]], [tables[l]], [adds[l]])
        assert torch.equal(one["y"][0], full["y"][l]), l
        assert torch.equal(one["idx"][0], full["idx"][l]), l
        if l + 1 < nl:
            xl = (one["y"][0] + adds[l + 1]).contiguous()
    _check_against_oracle(layers[:3], x, logits[:3], adds[:3],
                          {k: v[:3] for k, v in full.items() if k != "ws"}, tabs[:3])


def test_stack_against_decode_layer():
    """One layer: the bits of moe_decode_layer (the same two kernels), with
    identical routing outputs."""
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    shape = synth.LayerShape(512, 10, 1024, 384, True)
    layers, tabs = _layers(0, shape, (synth.FMT_Q2SM,), 0.8, dev)
    tab = torch.tensor(tabs[0], dtype=torch.int32, device=dev)
    T = 4
    x, logits, adds = _inputs(0, shape, T, 1, dev, sigma=1.5, step=7)
    out = _run(layers, x, logits, [tab], adds)
    y, idx, w, slot, me, mp, nm = bf.decode_layer(layers[0].layer_obj, x, logits[0], tab)
    torch.cuda.synchronize()
    assert torch.equal(out["idx"][0], idx) and torch.equal(out["w"][0], w)
    assert torch.equal(out["slot"][0], slot) and torch.equal(out["n_miss"][0][:2], nm[:2])
    assert torch.equal(out["y"][0], y)


def test_stack_graph_replays():
    """Captured in a graph: every replay (inputs refreshed between replays)
    equals the eager call on the same inputs."""
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    shape = synth.LayerShape(128, 6, 256, 128, True)
    fmts = (synth.FMT_Q2SM, synth.FMT_Q3G, synth.FMT_Q2SM)
    layers, tabs = _layers(0, shape, fmts, 0.8, dev)
    tables = [torch.tensor(t, dtype=torch.int32, device=dev) for t in tabs]
    T = 1
    x, logits, adds = _inputs(0, shape, T, len(fmts), dev, sigma=1.0, step=1)
    objs = [L.layer_obj for L in layers]
    ws = bf.new_stack_workspace(objs, T)
    ys = torch.empty((len(fmts), T, shape.d_model), dtype=torch.float32, device=dev)
    lg = torch.stack(logits)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        bf.decode_stack(objs, x, lg, tables, addends=adds, ys=ys, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bf.decode_stack(objs, x, lg, tables, addends=adds, ys=ys, ws=ws)
    for step in range(3):
        xs, lgs, _ = _inputs(0, shape, T, len(fmts), dev, sigma=1.0, step=10 + step)
        x.copy_(xs)
        lg.copy_(torch.stack(lgs))
        ys.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = ys.clone()
        eager = _run(layers, x, list(lg), tables, adds)
        assert torch.equal(got, eager["y"]), step


@pytest.mark.parametrize("E,k", [(300, 12), (512, 10), (1024, 16), (64, 16)])
def test_stack_routing_edge_cases(E, k):
    """Equal logits (ties go to the smaller expert id, more than 64 keys tied
    at the bound), NaN (ranks as -inf), -0.0 against +0.0, infinities, and two
    halves of 512 experts: routing outputs equal the oracle's, y within the bar."""
    dev = need_gpu()
    shape = synth.LayerShape(E, k, 128, 64, True)
    layers, tabs = _layers(0, shape, (synth.FMT_Q2SM, synth.FMT_Q3G), 0.9, dev)
    tables = [torch.tensor(t, dtype=torch.int32, device=dev) for t in tabs]
    T = 4
    x, _, adds = _inputs(0, shape, T, 2, dev, sigma=1.0, step=2)
    lg = torch.zeros((T, E))
    lg[0] = 1.0                                    # all equal: ids 0..k-1
    lg[1, ::7] = 2.0                               # ties spread over groups and halves
    lg[1, 5] = float("nan")
    lg[2, :E // 3] = -1.0
    lg[2, E // 3:E // 3 + 10] = -0.0
    lg[2, E // 2:E // 2 + 5] = 0.0
    lg[2, E - 1] = float("inf")
    lg[3] = torch.arange(E, dtype=torch.float32).flip(0) % 17
    lg2 = synth.make_logits(0, 9, T, E, 1.5)
    lg2[1, 3] = float("-inf")
    logits = [lg.to(dev), lg2.to(dev)]
    out = _run(layers, x, logits, tables, adds)
    _check_against_oracle(layers, x, logits, adds, out, tabs)
    assert list(out["idx"][0][0].cpu().numpy()) == list(range(k))


@pytest.mark.parametrize("T", [1, 4])
def test_stack_full_size_equals_one_layer_calls(T):
    """At the model's shape, 8 stacked layers (Q2SM and Q3G in turn) in one
    call give the bits of 8 one-layer calls chained here with the same fp32
    additions, with the routing outputs given per layer or not at all (the
    workspace's stand-ins then serve every layer)."""
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    shape = synth.config_shape(1)
    nl = 8
    fmts = [(synth.FMT_Q2SM, synth.FMT_Q3G)[l % 2] for l in range(nl)]
    x, logits, adds = _inputs(1, shape, T, nl, dev, sigma=1.5, step=11)
    only = [set(oracle.route_topk(logits[l].cpu().numpy(), shape.top_k)[0].reshape(-1).tolist())
            for l in range(nl)]
    layers, tabs = _layers(1, shape, fmts, 1.0, dev, only=only)
    tables = [torch.tensor(t, dtype=torch.int32, device=dev) for t in tabs]
    full = _run(layers, x, logits, tables, adds)
    objs = [L.layer_obj for L in layers]
    bare = bf.decode_stack(objs, x, logits, tables, addends=adds)   # no routing outputs
    torch.cuda.synchronize()
    assert torch.equal(bare["y"], full["y"])
    xl = x
    for l in range(nl):
        one = _run([layers[l]], xl, [logits[l]], [tables[l]], [adds[l]])
        assert torch.equal(one["y"][0], full["y"][l]), l
        assert torch.equal(one["idx"][0], full["idx"][l]), l
        assert torch.equal(one["w"][0], full["w"][l]), l
        if l + 1 < nl:
            xl = (one["y"][0] + adds[l + 1]).contiguous()
    _check_against_oracle(layers[:2], x, logits[:2], adds[:2],
                          {k: v[:2] for k, v in full.items() if k != "ws"}, tabs[:2])


def test_stack_cache_full_size_t4():
    """The expert-cache workload's shape through a stack at T = 4: 94 of 512
    experts + the shared one resident per layer (the seeded residency),
    Zipf(1.1) routing; every layer's routing outputs and miss lists exact,
    y (the resident part) within the bar."""
    dev = need_gpu()
    shape = synth.config_shape(2)
    c = synth.WORKLOADS[2]
    T, nl = 4, 3
    layers, tabs = [], []
    for l in range(nl):
        _, _, slot_expert = synth.make_slot_table(2, l)
        resident = [e for e in slot_expert if e < shape.n_experts]
        L = GpuLayer(2, l, shape, (synth.FMT_Q2SM, synth.FMT_Q3G)[l % 2], dev, resident=resident)
        layers.append(L)
        tabs.append(L.table)
    tables = [torch.tensor(t, dtype=torch.int32, device=dev) for t in tabs]
    x = synth.make_x(2, 0, T, shape.d_model).to(dev)
    logits = [synth.zipf_gumbel_logits(2, l, T, shape.n_experts, c["zipf_s"], step=5).to(dev)
              for l in range(nl)]
    adds = [0.5 * synth.make_x(2, 200 + l, T, shape.d_model).to(dev) for l in range(nl)]
    out = _run(layers, x, logits, tables, adds)
    nm = out["n_miss"].cpu().numpy()
    assert (nm[:, 1] > 0).all() and (nm[:, 1] < T * shape.top_k).all()   # hits and misses mixed
    _check_against_oracle(layers, x, logits, adds, out, tabs)
