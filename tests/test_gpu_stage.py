"""GPU parity: prefill with the layer staged from the GPU cache and the host
tier (moe_stage_layer).

The staging pool must hold exactly every expert's bytes in expert order, and
a prefill chunk run on it must give the same bits as on a pool that holds
every expert resident (at other slots), also when the staging of the next
layer runs on a second stream during the current layer's prefill; at full
size its y is also checked against the oracle on sampled tokens.
"""
import numpy as np
import pytest
import torch

import synth
from parity import need_gpu

pytestmark = pytest.mark.gpu


class TwoTierLayer:
    """Every expert of a layer: a full device pool at a permuted slot order
    (the reference), a GPU cache holding `n_res` of them plus the shared
    expert at other slots, and a pinned host tier at a third order."""

    def __init__(self, layer, shape, fmt, n_res, dev, seed=0):
        import bit_expert_ffn_top_amd as bf
        E = shape.n_experts
        rng = np.random.default_rng(900 + seed)
        ids = list(range(E)) + ([E] if shape.shared else [])
        packed = synth.make_layer_pool(4, layer, ids, device=dev, fmt=fmt, shape=shape)
        # reference: all resident, permuted
        order = rng.permutation(len(ids))
        self.full_pool = torch.empty_like(packed)
        self.full_pool[torch.tensor(order, device=dev)] = packed
        self.full_table = np.asarray(order[:E], np.int32)
        self.full = bf.MoeLayer(shape.d_model, shape.d_ff, E, shape.top_k, fmt, self.full_pool,
                                int(order[E]) if shape.shared else -1)
        # cache: n_res experts + shared
        res = np.sort(rng.choice(E, n_res, replace=False))
        n_slots = n_res + (1 if shape.shared else 0) + 3          # 3 empty slots
        slots = rng.permutation(n_slots)
        self.cache_pool = torch.zeros((n_slots, packed.shape[1]), dtype=torch.uint8, device=dev)
        self.slot_of_expert = np.full(E, -1, np.int32)
        for j, e in enumerate(res):
            self.slot_of_expert[e] = slots[j]
            self.cache_pool[int(slots[j])] = packed[e]
        shared_slot = -1
        if shape.shared:
            shared_slot = int(slots[n_res])
            self.cache_pool[shared_slot] = packed[E]
        self.cache = bf.MoeLayer(shape.d_model, shape.d_ff, E, shape.top_k, fmt, self.cache_pool,
                                 shared_slot)
        # host tier: every expert at yet another order
        horder = rng.permutation(E)
        self.host_slot = np.empty(E, np.int32)
        self.host_slot[horder] = np.arange(E, dtype=np.int32)
        host = torch.empty((E, packed.shape[1]), dtype=torch.uint8, pin_memory=True)
        pc = packed.cpu()
        for e in range(E):
            host[int(self.host_slot[e])] = pc[e]
        self.tier = bf.HostTier(shape.d_model, shape.d_ff, E, shape.top_k, fmt, host)
        self.packed = packed
        self.E = E


def _prefill(bf, L, x, logits, table, k, ws=None):
    idx, w = bf.route_topk(logits, k)
    slot, _, _, _ = bf.cache_lookup(idx, table)
    out_pairs, pair_pos, offs, out_sh = bf.expert_ffn_prefill(L, x, idx, slot,
                                                              with_shared=L.shared_slot >= 0)
    y = bf.combine(x, out_pairs, pair_pos, w, out_sh)
    return out_pairs, pair_pos, offs, out_sh, y


@pytest.mark.parametrize("fmt,shared", [(synth.FMT_Q2SM, True), (synth.FMT_Q3G, False)])
def test_stage_bytes_and_prefill_bitwise(fmt, shared):
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    shape = synth.LayerShape(64, 4, 256, 128, shared)
    Lr = TwoTierLayer(2, shape, fmt, 20, dev)
    E, k, T = shape.n_experts, shape.top_k, 300
    sb = Lr.packed.shape[1]
    staging = torch.full((E + 1, sb), 0x5A, dtype=torch.uint8, device=dev)
    S = bf.stage_layer(Lr.cache, Lr.slot_of_expert, Lr.tier, Lr.host_slot, staging)
    torch.cuda.synchronize()
    assert torch.equal(staging[:E], Lr.packed[:E])
    if shared:
        assert torch.equal(staging[E], Lr.packed[E])
    else:
        assert (staging[E] == 0x5A).all()                 # untouched without a shared expert
    x = synth.make_x(4, 2, T, shape.d_model, device=dev, dtype=torch.bfloat16)
    logits = synth.make_logits(4, 2, T, E, 1.5, device=dev)
    ident = torch.arange(E, dtype=torch.int32, device=dev)
    got = _prefill(bf, S, x, logits, ident, k)
    ref = _prefill(bf, Lr.full, x, logits, torch.tensor(Lr.full_table, device=dev), k)
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        if g is None:
            assert r is None
            continue
        assert torch.equal(g, r)


def test_staged_pipeline_two_streams():
    """Three layers; the staging of layer l+1 runs on its own stream while
    layer l's prefill runs (two staging buffers).  Every layer's output
    equals the all-resident prefill bit for bit."""
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    shape = synth.LayerShape(96, 6, 512, 256, True)
    E, k, T, n_layers = shape.n_experts, shape.top_k, 1000, 3
    layers = [TwoTierLayer(l, shape, synth.FMT_Q2SM, 30, dev, seed=l) for l in range(n_layers)]
    sb = layers[0].packed.shape[1]
    xs = [synth.make_x(4, l, T, shape.d_model, device=dev, dtype=torch.bfloat16)
          for l in range(n_layers)]
    lgs = [synth.make_logits(4, l, T, E, 1.5, device=dev) for l in range(n_layers)]
    ident = torch.arange(E, dtype=torch.int32, device=dev)
    refs = [_prefill(bf, L.full, xs[l], lgs[l], torch.tensor(L.full_table, device=dev), k)[4]
            for l, L in enumerate(layers)]
    torch.cuda.synchronize()
    staging = [torch.empty((E + 1, sb), dtype=torch.uint8, device=dev) for _ in range(2)]
    up = torch.cuda.Stream()
    comp = torch.cuda.current_stream()
    ev_up = [torch.cuda.Event() for _ in range(n_layers)]
    ev_done = [torch.cuda.Event() for _ in range(n_layers)]
    outs = []
    for l, L in enumerate(layers):
        with torch.cuda.stream(up):
            if l >= 2:
                up.wait_event(ev_done[l - 2])
            S = bf.stage_layer(L.cache, L.slot_of_expert, L.tier, L.host_slot, staging[l % 2],
                               stream=up)
            ev_up[l].record(up)
        comp.wait_event(ev_up[l])
        y = _prefill(bf, S, xs[l], lgs[l], ident, k)[4]
        outs.append(y.clone())
        ev_done[l].record(comp)
    torch.cuda.synchronize()
    for l in range(n_layers):
        assert torch.equal(outs[l], refs[l]), l


def test_stage_refuses_expert_without_source():
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    shape = synth.LayerShape(16, 2, 64, 32, True)
    Lr = TwoTierLayer(1, shape, synth.FMT_Q2S, 4, dev)
    hs = Lr.host_slot.copy()
    missing = int(np.nonzero(Lr.slot_of_expert < 0)[0][0])
    hs[missing] = -1
    sb = Lr.packed.shape[1]
    staging = torch.zeros((17, sb), dtype=torch.uint8, device=dev)
    with pytest.raises(bf.MoeError):
        bf.stage_layer(Lr.cache, Lr.slot_of_expert, Lr.tier, hs, staging)
    with pytest.raises(bf.MoeError):                      # staging one slot short
        bf.stage_layer(Lr.cache, Lr.slot_of_expert, Lr.tier, Lr.host_slot, staging[:16])
    torch.cuda.synchronize()
    assert not staging.any()                              # nothing was copied


def test_stage_full_size_bitwise():
    """The prefill workload's layer (E=512 + shared, d=2048, d_ff=768, Q2SM,
    T=8192): 94 experts resident, the other 418 staged from pinned host
    memory; the prefill on the staged pool equals the all-resident one bit
    for bit (pair rows, shared rows, y)."""
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    shape = synth.config_shape(4)
    T = synth.WORKLOADS[4]["T"]
    E, k = shape.n_experts, shape.top_k
    Lr = TwoTierLayer(5, shape, synth.FMT_Q2SM, 94, dev, seed=7)
    sb = Lr.packed.shape[1]
    staging = torch.empty((E + 1, sb), dtype=torch.uint8, device=dev)
    S = bf.stage_layer(Lr.cache, Lr.slot_of_expert, Lr.tier, Lr.host_slot, staging)
    x = synth.make_x(4, 5, T, shape.d_model, device=dev, dtype=torch.bfloat16)
    logits = synth.make_logits(4, 5, T, E, 1.5, device=dev)
    ident = torch.arange(E, dtype=torch.int32, device=dev)
    got = _prefill(bf, S, x, logits, ident, k)
    torch.cuda.synchronize()
    assert torch.equal(staging, Lr.packed)
    ref = _prefill(bf, Lr.full, x, logits, torch.tensor(Lr.full_table, device=dev), k)
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        assert torch.equal(g, r)
    # y of the staged prefill against the oracle on 16 seeded tokens (each
    # chosen expert unpacked once from its packed bytes, in worker processes)
    import oracle
    import oracle_pool
    from parity import check_close
    sample = np.sort(np.random.default_rng(5).choice(T, 16, replace=False))
    lg = logits.cpu().numpy()[sample]
    ridx, rw = oracle.route_topk(lg, k)
    xd = x.cpu().double().numpy()[sample]
    host = Lr.packed.cpu().numpy()
    experts = sorted(set(int(e) for e in ridx.reshape(-1))) + [E]
    tasks = [(host[e], xd) for e in experts]
    outs = dict(zip(experts, oracle_pool.ffn_rows_many(tasks, synth.FMT_Q2SM, shape.d_model,
                                                        shape.d_ff)))
    yref = xd + outs[E]
    for j in range(len(sample)):
        for i in range(k):
            yref[j] += rw[j, i] * outs[int(ridx[j, i])][j]
    check_close(got[4].cpu().numpy()[sample], yref, xd, what="staged prefill y")
