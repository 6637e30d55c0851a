"""GPU parity: prefill chunk (grouping, two grouped bf16 MFMA GEMMs, combine)
and the standalone combine, against the oracle.

expert_offsets and pair_pos must match bit for bit; out_pairs, out_shared
and y within max|err| <= 2e-3 max|ref| and normwise 1e-4 (on y and y - x).
The oracle rounds x, the dequantized weights and h = silu(g) * u to bf16 as
the kernels do."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import GpuLayer, check_close, need_gpu

pytestmark = pytest.mark.gpu


def _prefill(L, x_bf16, logits, k, dev, table=None, with_shared=True):
    import bit_expert_ffn_top_amd as bf
    idx, w = bf.route_topk(logits.to(dev), k)
    tab = L.table_dev(dev) if table is None else torch.tensor(table, dtype=torch.int32, device=dev)
    slot, _, _, _ = bf.cache_lookup(idx, tab)
    out_pairs, pair_pos, offs, out_sh = bf.expert_ffn_prefill(L.layer_obj, x_bf16.to(dev), idx,
                                                              slot, with_shared=with_shared)
    y = bf.combine(x_bf16.to(dev), out_pairs, pair_pos, w, out_sh)
    torch.cuda.synchronize()
    return (out_pairs.cpu(), pair_pos.cpu().numpy(), offs.cpu().numpy(),
            None if out_sh is None else out_sh.cpu(), y.cpu(), idx.cpu().numpy(),
            slot.cpu().numpy(), w.cpu().numpy())


def _oracle_groups(idx, slot, E):
    """Oracle grouping of the hit pairs only (misses get position -1)."""
    T, k = idx.shape
    hit = slot >= 0
    order = sorted((p for p in range(T * k) if hit.reshape(-1)[p]),
                   key=lambda p: (idx.reshape(-1)[p], p))
    counts = np.zeros(E, np.int64)
    for p in order:
        counts[idx.reshape(-1)[p]] += 1
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    pos = np.full(T * k, -1, np.int32)
    pos[np.array(order, dtype=np.int64)] = np.arange(len(order), dtype=np.int32)
    return offs, pos.reshape(T, k), order


CASES = [
    ("q2sm_T16", synth.LayerShape(64, 4, 256, 128, True), synth.FMT_Q2SM, 16),
    ("q2sm_T300", synth.LayerShape(64, 4, 256, 128, True), synth.FMT_Q2SM, 300),
    ("q2s_T130_noshared", synth.LayerShape(64, 4, 256, 128, False), synth.FMT_Q2S, 130),
    ("q3g_T77", synth.LayerShape(32, 6, 256, 192, True), synth.FMT_Q3G, 77),
    ("q2sm_T1", synth.LayerShape(64, 4, 256, 128, True), synth.FMT_Q2SM, 1),
    # smallest and largest sizes the prefill accepts: d_model 128 / d_ff 64,
    # and d_model 2048 / d_ff 4096 (64 down K steps, 16 gate/up column jobs)
    ("q2s_d128_f64", synth.LayerShape(16, 3, 128, 64, True), synth.FMT_Q2S, 50),
    ("q2sm_d2048_f4096", synth.LayerShape(6, 2, 2048, 4096, True), synth.FMT_Q2SM, 70),
]


@pytest.mark.parametrize("name,shape,fmt,T", CASES, ids=[c[0] for c in CASES])
def test_prefill_small(name, shape, fmt, T):
    dev = need_gpu()
    L = GpuLayer(4, 1, shape, fmt, dev, shared=shape.shared)
    x = synth.make_x(4, 1, T, shape.d_model, dtype=torch.bfloat16)
    logits = synth.make_logits(4, 1, T, shape.n_experts, 1.5)
    out_pairs, pair_pos, offs, out_sh, y, idx, slot, w = _prefill(L, x, logits, shape.top_k, dev)
    ridx, rw = oracle.route_topk(logits.numpy(), shape.top_k)
    np.testing.assert_array_equal(idx, ridx)
    roffs, rpos, _ = _oracle_groups(ridx, slot, shape.n_experts)
    np.testing.assert_array_equal(offs, roffs)
    np.testing.assert_array_equal(pair_pos, rpos)
    xd = x.double().numpy()
    shared_w = L.weights_of_slot(L.shared_slot) if shape.shared else None
    ro, rsh, ry = oracle.prefill_layer(xd, ridx, rw, L.weights_of_expert, shared_w, shape.n_experts)
    n = int(roffs[-1])
    check_close(out_pairs.numpy()[:n], ro[:n], what="out_pairs")
    if shape.shared:
        check_close(out_sh.numpy(), rsh, what="out_shared")
    check_close(y.numpy(), ry, xd)


def test_prefill_q2sm_tiny_min():
    """Q2SM blocks whose min is tiny next to the scale (|m| = s/2048), on
    every other block, beside ordinary ones: a dequantization that folded
    the min into an offset (m - c*s) would round there; the GEMMs must still
    match the oracle."""
    dev = need_gpu()
    shape = synth.LayerShape(64, 4, 256, 128, True)
    fmt = synth.FMT_Q2SM
    L = GpuLayer(4, 3, shape, fmt, dev)
    lay = synth.slot_layout(fmt, shape.d_model, shape.d_ff)
    host = L.pool.cpu().numpy()
    for mat in ("G", "D"):
        s_off, s_len = lay[(mat, "scale")]
        m_off, m_len = lay[(mat, "min")]
        scale = host[:, s_off:s_off + s_len].copy().view(np.float16).astype(np.float32)
        mins = host[:, m_off:m_off + m_len].copy().view(np.float16)
        tiny = (scale * np.float32(2.0 ** -11)).astype(np.float16)
        sign = np.where(np.arange(mins.shape[1]) % 4 == 0, -1, 1).astype(np.float16)
        mins[:, ::2] = tiny[:, ::2] * sign[::2]
        host[:, m_off:m_off + m_len] = mins.view(np.uint8)
    L.pool.copy_(torch.from_numpy(host).to(dev))
    L._bytes = {s_: host[s_] for s_ in L._bytes}
    L._w = {}
    T = 96
    x = synth.make_x(4, 3, T, shape.d_model, dtype=torch.bfloat16)
    logits = synth.make_logits(4, 3, T, shape.n_experts, 1.5)
    out_pairs, pair_pos, offs, out_sh, y, idx, slot, w = _prefill(L, x, logits, shape.top_k, dev)
    ridx, rw = oracle.route_topk(logits.numpy(), shape.top_k)
    np.testing.assert_array_equal(idx, ridx)
    xd = x.double().numpy()
    ro, rsh, ry = oracle.prefill_layer(xd, ridx, rw, L.weights_of_expert,
                                       L.weights_of_slot(L.shared_slot), shape.n_experts)
    n = int(offs[-1])
    check_close(out_pairs.numpy()[:n], ro[:n], what="out_pairs")
    check_close(out_sh.numpy(), rsh, what="out_shared")
    check_close(y.numpy(), ry, xd)


def test_prefill_with_misses():
    dev = need_gpu()
    shape = synth.LayerShape(64, 4, 256, 128, True)
    rng = np.random.default_rng(3)
    resident = np.sort(rng.choice(64, 40, replace=False))
    L = GpuLayer(4, 2, shape, synth.FMT_Q2SM, dev, resident=resident)
    T = 200
    x = synth.make_x(4, 2, T, 256, dtype=torch.bfloat16)
    logits = synth.make_logits(4, 2, T, 64, 1.5)
    out_pairs, pair_pos, offs, out_sh, y, idx, slot, w = _prefill(L, x, logits, 4, dev)
    assert (slot < 0).any()
    roffs, rpos, _ = _oracle_groups(idx, slot, 64)
    np.testing.assert_array_equal(offs, roffs)
    np.testing.assert_array_equal(pair_pos, rpos)
    # reference: per token, resident experts only, bf16 rounding points
    xd = x.double().numpy()
    ref = xd.copy()
    for t in range(T):
        for i in range(4):
            if slot[t, i] >= 0:
                ref[t] += w[t, i].astype(np.float64) * oracle.expert_ffn_bf16(
                    xd[t:t + 1], *L.weights_of_slot(int(slot[t, i])))[0]
        ref[t] += oracle.expert_ffn_bf16(xd[t:t + 1], *L.weights_of_slot(L.shared_slot))[0]
    check_close(y.numpy(), ref, xd)


def test_prefill_full_chunk_sampled():
    """The prefill chunk at full size: T=8192, E=512, top-10 + shared,
    d=2048, d_ff=768, Q2SM.  Grouping is checked in full; against the oracle
    (one expert unpacked at a time, in worker processes): all 8,192 shared
    rows, every pair row of 32 whole expert groups (the largest, the
    smallest and 30 seeded others), and y on 256 seeded tokens; y of every
    token equals the oracle's combine of the kernel's own rows."""
    import oracle_pool
    dev = need_gpu()
    shape = synth.config_shape(4)
    T, k, E, d, f = 8192, shape.top_k, shape.n_experts, shape.d_model, shape.d_ff
    L = GpuLayer(4, 0, shape, synth.FMT_Q2SM, dev)
    x = synth.make_x(4, 0, T, d, dtype=torch.bfloat16)
    logits = synth.make_logits(4, 0, T, E, 1.5)
    out_pairs, pair_pos, offs, out_sh, y, idx, slot, w = _prefill(L, x, logits, k, dev)
    ref_idx = np.argsort(-logits.numpy(), axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(idx, ref_idx)
    roffs, rpos, order = _oracle_groups(idx, slot, E)
    np.testing.assert_array_equal(offs, roffs)
    np.testing.assert_array_equal(pair_pos, rpos)
    xd = x.double().numpy()
    op = out_pairs.numpy()
    yg = y.numpy()
    osh_ref = oracle.expert_ffn_bf16(xd, *L.weights_of_slot(L.shared_slot))
    check_close(out_sh.numpy(), osh_ref, what="out_shared (all 8192 rows)")
    # the combine step on every token, over the kernel's own rows
    _, rw = oracle.route_topk(logits.numpy(), k)
    ycomb = oracle.combine(xd, op.astype(np.float64), pair_pos, rw, out_sh.numpy().astype(np.float64))
    check_close(yg, ycomb, xd, what="y vs combine of the kernel's rows")

    sizes = np.diff(offs)
    nonempty = np.flatnonzero(sizes > 0)
    big, small = int(nonempty[np.argmax(sizes[nonempty])]), int(nonempty[np.argmin(sizes[nonempty])])
    rng = np.random.default_rng(11)
    others = [int(e) for e in rng.permutation(nonempty) if e not in (big, small)][:30]
    groups = [big, small] + others
    flat = idx.reshape(-1)
    tokens_of = {e: np.array([p // k for p in order[offs[e]:offs[e + 1]]]) for e in groups}
    sample = np.sort(rng.choice(T, 256, replace=False))
    need = sorted(set(groups) | set(int(e) for e in idx[sample].reshape(-1)))
    tasks, keys = [], []
    for e in need:
        rows_t = tokens_of[e] if e in tokens_of else np.array([], dtype=np.int64)
        samp_t = sample[(idx[sample] == e).any(axis=1)]
        toks = np.unique(np.concatenate([rows_t, samp_t])).astype(np.int64)
        tasks.append((L._bytes[int(L.table[e])], xd[toks]))
        keys.append((e, toks))
    outs = oracle_pool.ffn_rows_many(tasks, L.fmt, d, f)
    ref_of = {}
    for (e, toks), o in zip(keys, outs):
        for t, row in zip(toks, o):
            ref_of[(e, int(t))] = row
    for e in groups:
        got = op[offs[e]:offs[e + 1]]
        ref = np.stack([ref_of[(e, int(t))] for t in tokens_of[e]])
        check_close(got, ref, what=f"out_pairs of group {e} ({len(ref)} rows)")
    yref = np.empty((len(sample), d))
    for j, t in enumerate(sample):
        acc = xd[t].copy()
        for i in range(k):
            acc += rw[t, i] * ref_of[(int(idx[t, i]), int(t))]
        yref[j] = acc + osh_ref[t]
    check_close(yg[sample], yref, xd[sample], what="y on 256 tokens")


def test_combine_parity():
    dev = need_gpu()
    import bit_expert_ffn_top_amd as bf
    rng = np.random.default_rng(7)
    T, d, k, R = 33, 512, 5, 200
    x = torch.tensor(rng.normal(size=(T, d)), dtype=torch.float32)
    rows = torch.tensor(rng.normal(size=(R, d)), dtype=torch.float32)
    pos = rng.choice(R, T * k, replace=False).reshape(T, k).astype(np.int32)
    pos[rng.random((T, k)) < 0.2] = -1
    w = torch.tensor(rng.random((T, k)), dtype=torch.float32)
    sh = torch.tensor(rng.normal(size=(T, d)), dtype=torch.float32)
    for xx in (x, x.to(torch.bfloat16)):
        for s in (sh, None):
            y = bf.combine(xx.to(dev), rows.to(dev), torch.tensor(pos, device=dev), w.to(dev),
                           None if s is None else s.to(dev))
            ref = oracle.combine(xx.double().numpy(), rows.double().numpy(), pos,
                                 w.double().numpy(), None if s is None else s.double().numpy())
            np.testing.assert_allclose(y.cpu().double().numpy(), ref, rtol=1e-5, atol=1e-5)


def test_prefill_skewed_groups():
    """Degenerate routing: one expert chosen first by every token (a group of
    600 rows: three 256-row tiles, the last ragged), one chosen by half of
    them (300 rows: two tiles), one never chosen (an empty group), and the
    rest spread; grouping exact, rows and y within the bar."""
    dev = need_gpu()
    shape = synth.LayerShape(16, 3, 256, 128, True)
    L = GpuLayer(4, 4, shape, synth.FMT_Q2SM, dev)
    T = 600
    x = synth.make_x(4, 4, T, shape.d_model, dtype=torch.bfloat16)
    logits = synth.make_logits(4, 4, T, shape.n_experts, 1.0)
    logits[:, 3] += 20.0                      # every token's first choice
    logits[: T // 2, 5] += 10.0               # second choice of half the tokens
    logits[:, 7] -= 50.0                      # never chosen
    out_pairs, pair_pos, offs, out_sh, y, idx, slot, w = _prefill(L, x, logits, shape.top_k, dev)
    ridx, rw = oracle.route_topk(logits.numpy(), shape.top_k)
    np.testing.assert_array_equal(idx, ridx)
    roffs, rpos, _ = _oracle_groups(ridx, slot, shape.n_experts)
    np.testing.assert_array_equal(offs, roffs)
    np.testing.assert_array_equal(pair_pos, rpos)
    sizes = np.diff(roffs)
    assert sizes[3] == T and sizes[5] >= T // 2 and sizes[7] == 0
    xd = x.double().numpy()
    ro, rsh, ry = oracle.prefill_layer(xd, ridx, rw, L.weights_of_expert,
                                       L.weights_of_slot(L.shared_slot), shape.n_experts)
    n = int(roffs[-1])
    check_close(out_pairs.numpy()[:n], ro[:n], what="out_pairs")
    check_close(out_sh.numpy(), rsh, what="out_shared")
    check_close(y.numpy(), ry, xd)
