"""GPU parity: the one-call decode layer (route + lookup + FFN).

Every output of moe_decode_layer must equal, bit for bit, what the three
separate calls (moe_route_topk, moe_cache_lookup, moe_expert_ffn_decode)
return for the same inputs; the routing outputs must also match the oracle
(indices exactly, weights to 1e-6), and y the oracle within the fp32 bounds.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import GpuLayer, check_close, need_gpu

pytestmark = pytest.mark.gpu


def _separate(L, x, logits, k, tab, dev):
    import bit_expert_ffn_top_amd as bf
    idx, w = bf.route_topk(logits, k)
    slot, me, mp, nm = bf.cache_lookup(idx, tab)
    y = bf.expert_ffn_decode(L.layer_obj, x, idx, slot, w)
    return y, idx, w, slot, me, mp, nm


def _compare(L, x, logits, table=None, oracle_check=True):
    import bit_expert_ffn_top_amd as bf
    dev = x.device
    k = L.shape.top_k
    tab = L.table_dev(dev) if table is None else torch.tensor(table, dtype=torch.int32, device=dev)
    got = bf.decode_layer(L.layer_obj, x, logits, tab)
    ref = _separate(L, x, logits, k, tab, dev)
    torch.cuda.synchronize()
    y, idx, w, slot, me, mp, nm = [t.cpu() for t in got]
    ry, ridx, rw, rslot, rme, rmp, rnm = [t.cpu() for t in ref]
    assert torch.equal(idx, ridx)
    assert torch.equal(w, rw)
    assert torch.equal(slot, rslot)
    assert torch.equal(nm[:2], rnm[:2])
    assert torch.equal(me[:int(nm[0])], rme[:int(rnm[0])])
    assert torch.equal(mp[:int(nm[1])], rmp[:int(rnm[1])])
    assert torch.equal(y, ry)
    if oracle_check:
        lg = logits.cpu().numpy()
        oidx, ow = oracle.route_topk(lg, k)
        np.testing.assert_array_equal(idx.numpy(), oidx)
        np.testing.assert_allclose(w.numpy(), ow, rtol=1e-6, atol=0)
        tabh = L.table if table is None else table
        oslot, ome, omp, onm = oracle.cache_lookup(oidx, tabh)
        np.testing.assert_array_equal(slot.numpy(), oslot)
        assert list(nm[:2].numpy()) == list(onm)
        np.testing.assert_array_equal(me[:onm[0]].numpy(), ome)
        np.testing.assert_array_equal(mp[:onm[1]].numpy(), omp)
        oy = oracle.layer_decode(x.cpu().double().numpy(), oidx, oslot, ow, L.weights_of_slot,
                                 L.shared_slot if L.shared_slot >= 0 else None)
        check_close(y.numpy(), oy, x.cpu().numpy())
    return idx.numpy(), slot.numpy()


CASES = [
    # name, shape, fmt, T, shared
    ("e64_q2s", synth.LayerShape(64, 4, 256, 128, False), synth.FMT_Q2S, 1, False),
    ("e100_q2sm_T3", synth.LayerShape(100, 5, 256, 128, True), synth.FMT_Q2SM, 3, True),
    ("e1024_q3g_T4_k16", synth.LayerShape(1024, 16, 128, 64, True), synth.FMT_Q3G, 4, True),
    ("e40_k1_T4", synth.LayerShape(40, 1, 512, 64, False), synth.FMT_Q2SM, 4, False),
    ("e1000_k64", synth.LayerShape(1000, 64, 64, 32, True), synth.FMT_Q2S, 1, True),
]


@pytest.mark.parametrize("name,shape,fmt,T,shared", CASES, ids=[c[0] for c in CASES])
def test_decode_layer_small(name, shape, fmt, T, shared):
    dev = need_gpu()
    L = GpuLayer(0, 4, shape, fmt, dev, shared=shared)
    x = synth.make_x(0, 4, T, shape.d_model).to(dev)
    logits = synth.make_logits(0, 4, T, shape.n_experts, 1.0).to(dev)
    _compare(L, x, logits)


@pytest.mark.parametrize("fmt,T", [(synth.FMT_Q2SM, 1), (synth.FMT_Q3G, 4), (synth.FMT_Q2S, 3),
                                   (synth.FMT_Q2SM, 2)])
def test_decode_layer_full_size(fmt, T):
    """E=512, top-10 + shared, d=2048, d_ff=768 (only the chosen experts'
    slots are filled; no other slot is read)."""
    dev = need_gpu()
    shape = synth.config_shape(1)
    x = synth.make_x(1, 1, T, shape.d_model)
    logits = synth.make_logits(1, 1, T, shape.n_experts, 1.5)
    ridx, _ = oracle.route_topk(logits.numpy(), shape.top_k)
    L = GpuLayer(1, 1, shape, fmt, dev, only_experts=set(ridx.reshape(-1).tolist()))
    _compare(L, x.to(dev), logits.to(dev))


def test_decode_layer_misses_zipf():
    """94 of 512 experts resident, Zipf routing: misses and hits mixed."""
    dev = need_gpu()
    shape = synth.config_shape(2)
    c = synth.WORKLOADS[2]
    table, _, slot_expert = synth.make_slot_table(2, 1)
    resident = [e for e in slot_expert if e < shape.n_experts]
    L = GpuLayer(2, 1, shape, synth.FMT_Q2SM, dev, resident=resident)
    T = 4
    x = synth.make_x(2, 1, T, shape.d_model)
    logits = synth.zipf_gumbel_logits(2, 1, T, shape.n_experts, c["zipf_s"])
    _, slot = _compare(L, x.to(dev), logits.to(dev))
    assert (slot < 0).any() and (slot >= 0).any()


def test_decode_layer_ties_nan_and_empty_cache():
    """Equal logits across and within groups of 64 (ties go to the smaller
    expert id), NaN (ranks as -inf), -0.0 vs +0.0, and a cache holding
    nothing (y = x + shared expert)."""
    dev = need_gpu()
    shape = synth.LayerShape(300, 12, 128, 64, True)
    L = GpuLayer(0, 6, shape, synth.FMT_Q2SM, dev)
    T = 4
    x = synth.make_x(0, 6, T, shape.d_model).to(dev)
    lg = torch.zeros((T, shape.n_experts))
    lg[0] = 1.0                                   # all equal: ids 0..11
    lg[1, ::7] = 2.0                              # ties spread over groups
    lg[1, 5] = float("nan")
    lg[2, 130:140] = -0.0
    lg[2, 200:205] = 0.0
    lg[2, :100] = -1.0
    lg[2, 299] = float("inf")
    lg[3] = torch.arange(shape.n_experts, dtype=torch.float32).flip(0) % 17
    idx, _ = _compare(L, x, lg.to(dev))
    assert list(idx[0]) == list(range(12))
    none = np.full(shape.n_experts, -1, np.int32)
    _, slot = _compare(L, x, lg.to(dev), table=none)
    assert (slot < 0).all()


def test_decode_layer_workspace_reuse():
    """One workspace through many calls of different T, each call bitwise
    equal to the three separate calls; graph replays equal the eager call."""
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    shape = synth.LayerShape(200, 8, 512, 256, True)
    L = GpuLayer(0, 12, shape, synth.FMT_Q2SM, dev)
    tab = L.table_dev(dev)
    k = shape.top_k
    ws = torch.empty((bf.decode_workspace_bytes(L.layer_obj, 4),), dtype=torch.uint8, device=dev)
    for step, T in enumerate((4, 1, 3, 1, 4, 2)):
        x = synth.make_x(0, 12, T, shape.d_model, step=step).to(dev)
        logits = synth.make_logits(0, 12, T, shape.n_experts, 1.0, step=step).to(dev)
        y, *_ = bf.decode_layer(L.layer_obj, x, logits, tab, ws=ws)
        ry, *_ = _separate(L, x, logits, k, tab, dev)
        torch.cuda.synchronize()
        assert torch.equal(y, ry), (step, T)
    # captured: replays equal the eager call
    T = 2
    x = synth.make_x(0, 12, T, shape.d_model, step=9).to(dev)
    logits = synth.make_logits(0, 12, T, shape.n_experts, 1.0, step=9).to(dev)
    out = dict(idx=torch.empty((T, k), dtype=torch.int32, device=dev),
               w=torch.empty((T, k), dtype=torch.float32, device=dev),
               slot=torch.empty((T, k), dtype=torch.int32, device=dev),
               miss_expert=torch.empty((T * k,), dtype=torch.int32, device=dev),
               miss_pair=torch.empty((T * k,), dtype=torch.int32, device=dev),
               n_miss=torch.empty((4,), dtype=torch.int32, device=dev),
               y=torch.empty((T, shape.d_model), dtype=torch.float32, device=dev))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        bf.decode_layer(L.layer_obj, x, logits, tab, ws=ws, **out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = out["y"].clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bf.decode_layer(L.layer_obj, x, logits, tab, ws=ws, **out)
    for _ in range(3):
        out["y"].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out["y"], eager)


def test_slots_outside_the_pool_are_misses():
    """Slot values at or past the pool's n_slots count as misses everywhere a
    pool is read: moe_decode_layer writes -1 for them and lists them as
    misses, moe_expert_ffn_decode skips them, moe_expert_ffn_prefill gives
    them pair_pos -1.  Every output equals, bit for bit, the same call with
    those entries set to -1."""
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    shape = synth.LayerShape(200, 8, 512, 256, True)
    L = GpuLayer(0, 13, shape, synth.FMT_Q2SM, dev)
    n_slots = L.pool.shape[0]
    k, T = shape.top_k, 4
    x = synth.make_x(0, 13, T, shape.d_model).to(dev)
    logits = synth.make_logits(0, 13, T, shape.n_experts, 1.0).to(dev)
    oidx, _ = oracle.route_topk(logits.cpu().numpy(), k)
    chosen = sorted(set(oidx.reshape(-1).tolist()))
    bad = chosen[::3]
    table_bad = L.table.copy()
    table_neg = L.table.copy()
    for j, e in enumerate(bad):
        table_bad[e] = (n_slots, n_slots + 7, 1 << 30, 2 ** 31 - 1)[j % 4]
        table_neg[e] = -1
    tb = torch.tensor(table_bad, dtype=torch.int32, device=dev)
    tn = torch.tensor(table_neg, dtype=torch.int32, device=dev)

    got = [t.cpu() for t in bf.decode_layer(L.layer_obj, x, logits, tb)]
    ref = [t.cpu() for t in bf.decode_layer(L.layer_obj, x, logits, tn)]
    y, idx, w, slot, me, mp, nm = got
    ry, ridx, rw, rslot, rme, rmp, rnm = ref
    assert torch.equal(idx, ridx) and torch.equal(w, rw)
    assert torch.equal(slot, rslot)
    assert all(int(s) == -1 for e, s in zip(idx.reshape(-1).tolist(), slot.reshape(-1).tolist())
               if e in bad)
    assert torch.equal(nm[:2], rnm[:2])
    assert set(bad) <= set(me[:int(nm[0])].tolist())
    assert torch.equal(me[:int(nm[0])], rme[:int(rnm[0])])
    assert torch.equal(mp[:int(nm[1])], rmp[:int(rnm[1])])
    assert torch.equal(y, ry)

    # given slots: the out-of-range values straight from the table
    idx_d = idx.to(dev)
    w_d = w.to(dev)
    slot_bad = tb[idx_d.long()]
    slot_neg = tn[idx_d.long()]
    yb = bf.expert_ffn_decode(L.layer_obj, x, idx_d, slot_bad, w_d)
    yn = bf.expert_ffn_decode(L.layer_obj, x, idx_d, slot_neg, w_d)
    torch.cuda.synchronize()
    assert torch.equal(yb.cpu(), yn.cpu())
    assert torch.equal(yb.cpu(), y)

    # prefill: the same pairs are misses
    xb = x.to(torch.bfloat16)
    pb = bf.expert_ffn_prefill(L.layer_obj, xb, idx_d, slot_bad)
    pn = bf.expert_ffn_prefill(L.layer_obj, xb, idx_d, slot_neg)
    torch.cuda.synchronize()
    out_b, pos_b, off_b = (t.cpu() for t in pb[:3])
    out_n, pos_n, off_n = (t.cpu() for t in pn[:3])
    assert torch.equal(pos_b, pos_n) and torch.equal(off_b, off_n)
    bad_pairs = np.isin(idx.numpy(), bad)
    assert (pos_b.numpy()[bad_pairs] == -1).all()
    n_rows = int(off_n[-1])
    assert torch.equal(out_b[:n_rows], out_n[:n_rows])
    if pb[3] is not None:
        assert torch.equal(pb[3].cpu(), pn[3].cpu())
