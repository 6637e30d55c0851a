"""fp64 oracle: what one routed-expert MoE layer computes.

Test infrastructure.  Not imported by the library.

Sources (page titles as printed on the pages):
  [P2] "Strataとは？VRAM 12GBのGPUでQwen3.8-Flash-Nextを動かす方法" (vramglass.com)
       sections "なぜVRAM 12GBで足りるのか", "その1", "その2", "その3".
  [P4] "Strata" (news.blueqat.app post 3262), sections "Strataとは",
       "GPU・CPU・RAM・SSDの分担", "投機的デコード", "量子化の種類とサイズ".
  [P1] "FreeToken vs Strata" (geekoyaji.com), section "共通の仕組み".

The pages fix the counts (48 layers, 512 experts per layer, 10 chosen per
token plus one shared expert: [P4] "Strataとは"), the split of a layer's
chosen experts into those resident on the GPU and those computed elsewhere
([P2] "その2"), the per-layer join of both parts ([P1] "共通の仕組み"),
verification of up to 3 drafted tokens in one pass whose output equals plain
decoding ([P2] "その3", [P4] "投機的デコード") and 8,192-token prefill chunks
([P4] "GPU・CPU・RAM・SSDの分担").  They give no formula; the readings used
where they are silent (SwiGLU experts, softmax over the k chosen logits,
shared expert with weight 1, block formats, tie order) are stated at each
function.

Every function here is pinned by the CPU tests against hand-built blocks
with closed-form values, brute-force enumeration, library routines or exact
invariants; none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

FMT_Q2S, FMT_Q2SM, FMT_Q3G = 1, 2, 3
_BLK = 32
_ALIGN = 256


# ---------------------------------------------------------------------------
# packed expert slots
# ---------------------------------------------------------------------------

def _plane_list(fmt):
    # (name, bytes per 32-weight block) in storage order
    return {
        FMT_Q2S: [("codes", 8), ("scale", 2)],
        FMT_Q2SM: [("codes", 8), ("scale", 2), ("min", 2)],
        FMT_Q3G: [("codes", 8), ("hi", 4), ("scale", 2)],
    }[fmt]


def plane_offsets(fmt, d_model, d_ff):
    """Byte offset of every plane of the two matrices inside one slot.

    G (2*d_ff x d_model, gate row j at 2j, up row j at 2j+1) comes first,
    then D (d_model x d_ff).  Planes are 256-byte aligned from the slot start;
    a plane holds per-block data (codes 8 B, hi 4 B, scale 2 B, min 2 B).
    """
    offs = {}
    pos = 0
    for mat, rows, cols in (("G", 2 * d_ff, d_model), ("D", d_model, d_ff)):
        nblocks = rows * cols // _BLK
        for name, per in _plane_list(fmt):
            offs[(mat, name)] = pos
            pos += nblocks * per
            pos = -(-pos // _ALIGN) * _ALIGN
    offs["end"] = pos
    return offs


def slot_size(fmt, d_model, d_ff):
    return plane_offsets(fmt, d_model, d_ff)["end"]


def _grid_q3g():
    # The 8-entry 3-bit grid: -3.5, -2.5, ..., 3.5 (times s/3.5).
    return np.array([-3.5, -2.5, -1.5, -0.5, 0.5, 1.5, 2.5, 3.5], dtype=np.float64)


def _hi_position(i):
    """Bit of the 32-bit hi word that holds bit 2 of code i of a block."""
    return 2 * i + 1 if i < 16 else 2 * (i - 16)


def unpack_matrix(slot, fmt, d_model, d_ff, which):
    """Dequantize matrix `which` ('G' or 'D') of one packed slot to float64.

    Block formats (2-3-bit block-quantized expert weights stand in for the
    2-3-bit files of [P4] "量子化の種類とサイズ"; the exact block layouts
    are this library's own):
      Q2S : w = s * (q - 1.5)              q = 2-bit code
      Q2SM: w = m + s * q                  q = 2-bit code, m = block min
      Q3G : w = s * grid[q] / 3.5          q = lo2 + 4 * hi1, grid above
    s, m are IEEE fp16 read exactly; every product and sum here is exact
    in float64 except the Q3G division by 3.5.

    Storage order: units of U blocks of one row (U = 2 for G, 1 for D);
    unit c of row r is the (c * rows + r)-th unit of every plane.
    """
    slot = np.asarray(slot, dtype=np.uint8).reshape(-1)
    rows, cols = (2 * d_ff, d_model) if which == "G" else (d_model, d_ff)
    nb = cols // _BLK
    U = 2 if which == "G" else 1
    nblocks = rows * nb
    offs = plane_offsets(fmt, d_model, d_ff)

    def plane(name, per):
        o = offs[(which, name)]
        raw = slot[o:o + nblocks * per].reshape(nb // U, rows, U, per)
        # -> blocks in row-major order: [row][block in row][bytes]
        return np.ascontiguousarray(raw.transpose(1, 0, 2, 3)).reshape(-1)

    word = plane("codes", 8).view("<u8").astype(np.uint64)          # [nblocks]
    shifts = (2 * np.arange(_BLK)).astype(np.uint64)
    q = ((word[:, None] >> shifts[None, :]) & np.uint64(3)).astype(np.int64)
    if fmt == FMT_Q3G:
        hiw = plane("hi", 4).view("<u4").astype(np.uint64)
        hpos = np.array([_hi_position(i) for i in range(_BLK)], dtype=np.uint64)
        bits = ((hiw[:, None] >> hpos[None, :]) & np.uint64(1)).astype(np.int64)
        q = q + 4 * bits
    s = plane("scale", 2).view("<f2").astype(np.float64)[:, None]
    if fmt == FMT_Q2S:
        w = s * (q.astype(np.float64) - 1.5)
    elif fmt == FMT_Q2SM:
        m = plane("min", 2).view("<f2").astype(np.float64)[:, None]
        w = m + s * q.astype(np.float64)
    elif fmt == FMT_Q3G:
        w = s * _grid_q3g()[q] / 3.5
    else:
        raise ValueError(fmt)
    return w.reshape(rows, cols)


def unpack_expert(slot, fmt, d_model, d_ff):
    """(W_gate [f,d], W_up [f,d], W_down [d,f]) in float64."""
    G = unpack_matrix(slot, fmt, d_model, d_ff, "G")
    D = unpack_matrix(slot, fmt, d_model, d_ff, "D")
    return G[0::2], G[1::2], D


# ---------------------------------------------------------------------------
# router projection (adjacent to the path)
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits):
    """Value of each bfloat16 bit pattern (uint16): the upper half of the
    IEEE single with the same sign, exponent and top 7 mantissa bits."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def router_logits(x, w_bits):
    """Router projection ([P2] "なぜVRAM 12GBで足りるのか" and [P4]
    "GPU・CPU・RAM・SSDの分担": the router is part of the common part that
    stays on the GPU; it turns a token's hidden state into one logit per
    routed expert).  The pages give no precision; the reading here: router
    weights stored as bfloat16, [E][d] row-major (w_bits, uint16), the hidden
    state and the logits in fp32, the sums exact (float64 here).
    x [T][d] -> logits [T][E] = x . W^T."""
    x = np.asarray(x, dtype=np.float64)
    W = bf16_bits_to_f64(w_bits)
    return x @ W.T


# ---------------------------------------------------------------------------
# router top-k
# ---------------------------------------------------------------------------

def _order_key(v):
    """Logit as used for ranking: NaN ranks as -inf; -0.0 equals +0.0."""
    v = float(v)
    if v != v:
        return -np.inf
    return v + 0.0


def route_topk(logits, k):
    """Per token: the k experts with the largest logits and their weights.

    [P4] "Strataとは": each token picks 10 of a layer's 512 experts.
    Reading: rank by (logit descending, expert index ascending), NaN ranks as
    -inf, -0.0 equals +0.0; weights are the softmax over the k chosen logits,
    w_i = exp(l_i - l_0) / sum_j exp(l_j - l_0) with l_0 the largest (a
    difference of two equal values, also of two equal infinities, is 0).
    Returns idx int32 [T,k] in rank order and w float64 [T,k].
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    idx = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        keys = [(-_order_key(logits[t, e]), e) for e in range(E)]
        keys.sort()
        chosen = [e for _, e in keys[:k]]
        vals = np.array([_order_key(logits[t, e]) for e in chosen], dtype=np.float64)
        with np.errstate(invalid="ignore"):
            diff = np.where(vals == vals[0], 0.0, vals - vals[0])
        ex = np.exp(diff)
        idx[t] = chosen
        w[t] = ex / ex.sum()
    return idx, w


# ---------------------------------------------------------------------------
# expert-cache lookup
# ---------------------------------------------------------------------------

def cache_lookup(idx, slot_of_expert):
    """Split the chosen experts into resident (hit) and not resident (miss).

    [P2] "その1"/"その2": the GPU holds a cache of the most used experts;
    chosen experts not in it are computed elsewhere, not copied over.
    slot[t,i] = slot_of_expert[idx[t,i]] (-1 = miss);
    miss_expert = ascending distinct missed expert ids;
    miss_pair   = t*k+i of every missed pair, ordered by (expert, t, i);
    n_miss      = [len(miss_expert), len(miss_pair)].
    """
    idx = np.asarray(idx, dtype=np.int64)
    table = np.asarray(slot_of_expert, dtype=np.int64)
    T, k = idx.shape
    slot = table[idx].astype(np.int32)
    pairs = []
    for t in range(T):
        for i in range(k):
            if slot[t, i] < 0:
                pairs.append((int(idx[t, i]), t, i))
    pairs.sort()
    miss_expert = np.array(sorted({e for e, _, _ in pairs}), dtype=np.int32)
    miss_pair = np.array([t * k + i for _, t, i in pairs], dtype=np.int32)
    n_miss = np.array([len(miss_expert), len(miss_pair)], dtype=np.int32)
    return slot, miss_expert, miss_pair, n_miss


# ---------------------------------------------------------------------------
# cache admission and eviction
# ---------------------------------------------------------------------------

def cache_count(counts, idx):
    """Usage counts: counts[e] plus the number of times expert e is chosen in
    idx ([P1] table "VRAMのエキスパートの入れ替え": the cache starts from a
    table of measured usage frequencies).  Returns a new uint32 array."""
    out = np.asarray(counts, dtype=np.uint64).copy()
    for e in np.asarray(idx).reshape(-1):
        out[int(e)] += 1
    return (out & 0xFFFFFFFF).astype(np.uint32)


def cache_plan(counts, slot_of_expert, expert_of_slot, shared_slot, host_slot, host_n_slots,
               max_swaps, decay_shift):
    """Choose which experts enter and leave the GPU cache.

    [P1] table "VRAMのエキスパートの入れ替え" and [P2] "その1": the cache holds
    the most used experts and is updated as the conversation moves on;
    [P4] "GPU・CPU・RAM・SSDの分担": the cache changes with the conversation.
    The pages give no rule; the reading used:

    * candidates: experts not resident (slot_of_expert < 0) with a copy in the
      host tier (0 <= host_slot < host_n_slots) and a count above 0, best
      first by (count descending, id ascending);
    * victims: the cache's slots except the shared expert's, worst first by
      (key ascending, slot ascending), where an empty slot
      (expert_of_slot = -1) has key -1 and a full one its expert's count;
    * the i-th candidate replaces the i-th victim while i < max_swaps and its
      count is strictly above the victim's key (equal counts never swap);
    * the evicted expert leaves the slot table at once
      (slot_of_expert[old] = -1) and the slot is reserved for the newcomer
      (expert_of_slot[slot] = new); the newcomer becomes visible only at
      cache_commit, after its bytes have been copied;
    * afterwards every count is shifted right by decay_shift, so that old
      use fades (halving per update for a shift of 1).

    Returns (counts, slot_of_expert, expert_of_slot, swaps) with swaps a list
    of (slot, old expert or -1, new expert, host slot of the new expert).
    """
    cnt = np.asarray(counts, dtype=np.int64)
    soe = np.asarray(slot_of_expert, dtype=np.int32).copy()
    eos = np.asarray(expert_of_slot, dtype=np.int32).copy()
    hs = np.asarray(host_slot, dtype=np.int64)
    E = len(cnt)
    cands = [e for e in range(E)
             if soe[e] < 0 and 0 <= hs[e] < host_n_slots and cnt[e] > 0]
    cands.sort(key=lambda e: (-cnt[e], e))
    victims = []
    for s in range(len(eos)):
        if s == shared_slot:
            continue
        key = -1 if eos[s] < 0 else int(cnt[eos[s]])
        victims.append((key, s))
    victims.sort()
    swaps = []
    for i in range(min(max_swaps, len(cands), len(victims))):
        e = cands[i]
        key, s = victims[i]
        if not cnt[e] > key:
            break
        old = int(eos[s])
        if old >= 0:
            soe[old] = -1
        eos[s] = e
        swaps.append((s, old, e, int(hs[e])))
    out = (cnt >> int(decay_shift)).astype(np.uint32)
    return out, soe, eos, swaps


def cache_commit(slot_of_expert, swaps):
    """The newcomers of a plan become visible: slot_of_expert[new] = slot."""
    soe = np.asarray(slot_of_expert, dtype=np.int32).copy()
    for s, _, e, _ in swaps:
        soe[e] = s
    return soe


# ---------------------------------------------------------------------------
# expert FFN and the layer
# ---------------------------------------------------------------------------

def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def expert_ffn(x, Wg, Wu, Wd):
    """One expert on rows x [T,d]: W_down (silu(W_gate x) * (W_up x)).

    Reading: the expert is a gated (SwiGLU) FFN with no biases; the pages
    name the expert FFN but not its form.
    """
    x = np.asarray(x, dtype=np.float64)
    g = x @ Wg.T
    u = x @ Wu.T
    return (silu(g) * u) @ Wd.T


def layer_decode(x, idx, slot, w, slot_weights, shared_slot, hits_only=True):
    """One layer for T tokens routed independently.

    y_t = x_t + sum_{i: chosen} w[t,i] * FFN_{idx[t,i]}(x_t) + FFN_shared(x_t).
    With hits_only the sum runs over resident experts only (slot >= 0): the
    GPU part of the split of [P2] "その2"; the rest is added by whoever
    computes the misses ([P1] "共通の仕組み").  The shared expert ([P4]
    "Strataとは", "10個と共有エキスパート1個") always runs with weight 1
    (reading: it has no gate of its own).
    `slot_weights(s)` returns (Wg, Wu, Wd) float64 of slot s.
    """
    x = np.asarray(x, dtype=np.float64)
    T, k = np.asarray(idx).shape
    y = x.copy()
    cache = {}

    def W(s):
        if s not in cache:
            cache[s] = slot_weights(s)
        return cache[s]

    for t in range(T):
        acc = np.zeros_like(x[t])
        for i in range(k):
            s = int(slot[t][i])
            if s < 0 and hits_only:
                continue
            acc += w[t][i] * expert_ffn(x[t:t + 1], *W(s))[0]
        if shared_slot is not None and shared_slot >= 0:
            acc += expert_ffn(x[t:t + 1], *W(int(shared_slot)))[0]
        y[t] = x[t] + acc
    return y


def layer_decode_tiers(x, idx, w, slot, slot_weights, shared_slot, host_slot, host_weights,
                       max_rank=None):
    """One layer whose chosen experts sit in two tiers: the GPU cache and a
    host-memory copy of the layer's experts.

    [P2] "その2" and [P1] "共通の仕組み": the resident experts run on the GPU,
    the misses are computed from host memory at the same time, and the two
    parts are joined before the next layer.  [P4] "どう見るか": a setting
    (on by default for NVIDIA GPUs from release 0.1.42) leaves out missed
    experts of low rank, which changes the output slightly.

    Readings: a miss's rank is its k-slot i (route_topk lists each token's
    experts by descending logit); with max_rank = r a miss runs only if
    i < r (None: every miss runs); the weights of the terms kept are not
    renormalised (the pages name no rescaling); a miss whose expert has no
    host slot (host_slot[e] < 0) contributes nothing.

    y_t = x_t + sum_i term(t, i) + FFN_shared(x_t), where term(t, i) is
      w[t,i] * FFN of GPU slot slot[t,i]          if slot[t,i] >= 0,
      w[t,i] * FFN of host slot host_slot[e]      if slot[t,i] < 0, i < r and
                                                  host_slot[e] >= 0 (e = idx[t,i]),
      0                                           otherwise.
    `slot_weights(s)` / `host_weights(h)` return (Wg, Wu, Wd) float64.
    """
    x = np.asarray(x, dtype=np.float64)
    idx = np.asarray(idx)
    T, k = idx.shape
    r = k if max_rank is None else int(max_rank)
    hs = np.asarray(host_slot)
    y = x.copy()
    for t in range(T):
        acc = np.zeros_like(x[t])
        for i in range(k):
            s = int(slot[t][i])
            if s >= 0:
                W = slot_weights(s)
            else:
                h = int(hs[int(idx[t, i])])
                if i >= r or h < 0:
                    continue
                W = host_weights(h)
            acc += w[t][i] * expert_ffn(x[t:t + 1], *W)[0]
        if shared_slot is not None and shared_slot >= 0:
            acc += expert_ffn(x[t:t + 1], *slot_weights(int(shared_slot)))[0]
        y[t] = x[t] + acc
    return y


def layer_dense_mixture(x, logits, expert_w, k, shared_w=None):
    """Dense definition: every one of the E experts evaluated, then only the
    top-k of each token kept with softmax weights.  Used to pin the sparse
    path (with k = E it is the plain softmax mixture of all experts).
    `expert_w` is a list of (Wg, Wu, Wd) per expert id.
    """
    x = np.asarray(x, dtype=np.float64)
    logits = np.asarray(logits, dtype=np.float32)
    T = x.shape[0]
    E = len(expert_w)
    out = np.stack([expert_ffn(x, *expert_w[e]) for e in range(E)], axis=1)  # [T,E,d]
    y = x.copy()
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-_order_key(logits[t, e]), e))[:k]
        l = np.array([_order_key(logits[t, e]) for e in order])
        with np.errstate(invalid="ignore"):
            p = np.exp(np.where(l == l[0], 0.0, l - l[0]))
        p /= p.sum()
        y[t] += (p[:, None] * out[t, order]).sum(0)
        if shared_w is not None:
            y[t] += expert_ffn(x[t:t + 1], *shared_w)[0]
    return y


def union_plan(idx, slot, shared_slot):
    """Verify step ([P2] "その3", [P4] "投機的デコード"): the distinct
    resident experts chosen by any of the T tokens, each listed once, in order
    of first appearance over (t, i), with the tokens that chose it; the
    shared expert last with all tokens.  Returns [(slot, [tokens])]."""
    T, k = np.asarray(idx).shape
    order = []
    tokens = {}
    for t in range(T):
        for i in range(k):
            s = int(slot[t][i])
            if s < 0:
                continue
            if s not in tokens:
                tokens[s] = []
                order.append(s)
            tokens[s].append(t)
    plan = [(s, tokens[s]) for s in order]
    if shared_slot is not None and shared_slot >= 0:
        plan.append((int(shared_slot), list(range(T))))
    return plan


# ---------------------------------------------------------------------------
# prefill chunk
# ---------------------------------------------------------------------------

def bf16_round(a):
    """Round float64 values to the nearest bfloat16 (ties to even), returned
    as float64.  bfloat16 keeps 8 significant bits; below 2^-126 the spacing
    is fixed at 2^-133."""
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)                      # a = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)
    ulp_exp = e - 8
    r = np.rint(np.ldexp(a, -ulp_exp))      # exact scaling by a power of two
    return np.ldexp(r, ulp_exp)


def expert_ffn_bf16(x_bf16, Wg, Wu, Wd):
    """Expert FFN with the prefill chunk's rounding points: activations and
    weights enter as bfloat16 values, products are summed exactly (float64
    here), h = silu(g) * u is rounded to bfloat16, the output stays wide."""
    x = np.asarray(x_bf16, dtype=np.float64)
    g = x @ bf16_round(Wg).T
    u = x @ bf16_round(Wu).T
    h = bf16_round(silu(g) * u)
    return h @ bf16_round(Wd).T


def permute_pairs(idx, n_experts):
    """Token-by-expert permutation for the grouped product.

    Every (t, i) pair goes to its expert's group; groups in expert order,
    inside a group by t then i.  Returns expert_offsets [E+1] (prefix sums of
    the group sizes), perm [T*k] (pair id t*k+i at each position) and
    pair_pos [T,k] (position of pair (t,i)); pair_pos[perm[p]] == p.
    """
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    order = sorted(range(T * k), key=lambda p: (idx[p // k, p % k], p))
    perm = np.array(order, dtype=np.int32)
    counts = np.bincount(idx.reshape(-1), minlength=n_experts)
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    pair_pos = np.empty(T * k, dtype=np.int32)
    pair_pos[perm] = np.arange(T * k, dtype=np.int32)
    return offsets, perm, pair_pos.reshape(T, k)


def prefill_layer(x_bf16, idx, w, expert_w, shared_w, n_experts):
    """One prefill chunk ([P4] "GPU・CPU・RAM・SSDの分担": up to 8,192
    tokens at a time), every chosen expert resident.

    Returns (out_pairs [T*k, d] in permuted order, out_shared [T,d], y [T,d])
    with the rounding points of expert_ffn_bf16 and the combine
    y_t = x_t + sum_i w[t,i] * out_pairs[pair_pos[t,i]] + out_shared[t].
    `expert_w(e)` returns (Wg, Wu, Wd) of expert e.
    """
    x = np.asarray(x_bf16, dtype=np.float64)
    T, k = np.asarray(idx).shape
    offsets, perm, pair_pos = permute_pairs(idx, n_experts)
    d = x.shape[1]
    out_pairs = np.zeros((T * k, d), dtype=np.float64)
    for e in range(n_experts):
        p0, p1 = offsets[e], offsets[e + 1]
        if p1 == p0:
            continue
        rows = perm[p0:p1] // k
        out_pairs[p0:p1] = expert_ffn_bf16(x[rows], *expert_w(e))
    out_shared = expert_ffn_bf16(x, *shared_w) if shared_w is not None else None
    y = combine(x, out_pairs, pair_pos, w, out_shared)
    return out_pairs, out_shared, y


def combine(x, rows, pair_pos, w, shared=None):
    """y_t = x_t + sum_i w[t,i] * rows[pair_pos[t,i]] + shared_t.

    pair_pos < 0 marks a pair whose row is not present (a miss); it adds
    nothing.  [P1] "共通の仕組み": the layer's parts are joined before the
    next layer.
    """
    x = np.asarray(x, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64)
    T, k = np.asarray(pair_pos).shape
    y = x.copy()
    for t in range(T):
        for i in range(k):
            p = int(pair_pos[t][i])
            if p >= 0:
                y[t] += w[t][i] * rows[p]
        if shared is not None:
            y[t] += np.asarray(shared, dtype=np.float64)[t]
    return y
