"""Host checks of the Python binding: tensors of the wrong shape are refused
with a ValueError naming the argument, before anything reaches the library
(so a wrong size never becomes an out-of-bounds access on the device).  The
tensors here live on the CPU; the shape checks come before the device checks.
"""
import numpy as np
import pytest
import torch

import bit_expert_ffn_top_amd as bf
import synth


def _raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def _layer(d=64, f=32, E=8, k=2):
    pool = torch.zeros((E + 1, synth.slot_bytes(synth.FMT_Q2SM, d, f)), dtype=torch.uint8)
    return bf.MoeLayer(d, f, E, k, synth.FMT_Q2SM, pool, E)


def test_route_topk_shapes():
    _raises(r"logits: shape", bf.route_topk, torch.zeros(8), 2)
    # right shape, wrong place: the device check speaks
    _raises(r"logits must be a device tensor", bf.route_topk, torch.zeros((2, 8)), 2)


def test_lookup_shapes():
    _raises(r"idx: shape", bf.cache_lookup, torch.zeros(4, dtype=torch.int32),
            torch.zeros(8, dtype=torch.int32))
    _raises(r"slot_of_expert: shape", bf.cache_lookup, torch.zeros((2, 2), dtype=torch.int32),
            torch.zeros((8, 1), dtype=torch.int32))


def test_decode_shapes():
    L = _layer()
    x = torch.zeros((1, 32))                                   # d_model is 64
    ids = torch.zeros((1, 2), dtype=torch.int32)
    _raises(r"x: shape \(\*, 64\)", bf.expert_ffn_decode, L, x, ids, ids, torch.zeros((1, 2)))
    _raises(r"x: shape \(\*, 64\)", bf.decode_layer, L, x, torch.zeros((1, 8)),
            torch.zeros(8, dtype=torch.int32))


def test_decode_misses_shapes():
    L = _layer()
    tier = bf.HostTier.__new__(bf.HostTier)        # shape fields only: no pool needed here
    tier.d_model, tier.d_ff, tier.n_experts, tier.top_k = L.d_model, L.d_ff, L.n_experts, L.top_k
    x = torch.zeros((1, 64))
    ids = torch.zeros((1, 2), dtype=torch.int32)
    w = torch.zeros((1, 2))
    _raises(r"host_slot_of_expert: shape \(8,\)", bf.decode_misses, tier, x, ids, ids, w,
            torch.zeros(7, dtype=torch.int32), torch.zeros((1, 64)))
    _raises(r"y: shape \(1, 64\)", bf.decode_misses, tier, x, ids, ids, w,
            torch.zeros(8, dtype=torch.int32), torch.zeros((2, 64)))
    _raises(r"idx: shape \(1, 2\)", bf.decode_misses, tier, x, torch.zeros((1, 3), dtype=torch.int32),
            ids, w, torch.zeros(8, dtype=torch.int32), torch.zeros((1, 64)))


def test_decode_layer_tiers_shapes():
    L = _layer()
    tier = bf.HostTier.__new__(bf.HostTier)        # shape fields only: no pool needed here
    tier.d_model, tier.d_ff, tier.n_experts, tier.top_k = L.d_model, L.d_ff, L.n_experts, L.top_k
    x = torch.zeros((1, 64))
    tab = torch.zeros(8, dtype=torch.int32)
    _raises(r"x: shape \(\*, 64\)", bf.decode_layer_tiers, L, tier, torch.zeros((1, 32)),
            torch.zeros((1, 8)), tab, tab)
    _raises(r"logits: shape \(1, 8\)", bf.decode_layer_tiers, L, tier, x, torch.zeros((2, 8)),
            tab, tab)
    _raises(r"slot_of_expert: shape \(8,\)", bf.decode_layer_tiers, L, tier, x,
            torch.zeros((1, 8)), torch.zeros(9, dtype=torch.int32), tab)
    _raises(r"host_slot_of_expert: shape \(8,\)", bf.decode_layer_tiers, L, tier, x,
            torch.zeros((1, 8)), tab, torch.zeros(7, dtype=torch.int32))
    _raises(r"x must be a device tensor", bf.decode_layer_tiers, L, tier, x,
            torch.zeros((1, 8)), tab, tab)


def test_cache_plan_shapes():
    i32 = dict(dtype=torch.int32)
    counts = torch.zeros(8, **i32)
    _raises(r"slot_of_expert: shape \(8,\)", bf.cache_plan, counts, torch.zeros(7, **i32),
            torch.zeros(4, **i32), -1, torch.zeros(8, **i32), 8, 2)
    _raises(r"host_slot_of_expert: shape \(8,\)", bf.cache_plan, counts, torch.zeros(8, **i32),
            torch.zeros(4, **i32), -1, torch.zeros(9, **i32), 8, 2)


def test_stage_layer_shapes():
    L = _layer()
    tier = bf.HostTier.__new__(bf.HostTier)
    _raises(r"slot_of_expert: shape \(8,\)", bf.stage_layer, L, np.zeros(7, np.int32), tier,
            np.zeros(8, np.int32), torch.zeros(1, dtype=torch.uint8))
    _raises(r"host_slot_of_expert: shape \(8,\)", bf.stage_layer, L, np.zeros(8, np.int32), tier,
            np.zeros(9, np.int32), torch.zeros(1, dtype=torch.uint8))


def test_prefill_shapes():
    L = _layer(d=128, f=64)
    ids = torch.zeros((3, 2), dtype=torch.int32)
    _raises(r"x_bf16: shape \(\*, 128\)", bf.expert_ffn_prefill, L,
            torch.zeros((3, 64), dtype=torch.bfloat16), ids, ids)


def test_combine_shapes():
    _raises(r"x: shape", bf.combine, torch.zeros(4), None, None, None)
