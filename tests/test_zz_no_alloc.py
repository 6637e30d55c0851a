"""GPU test of moe_decode_layer_noalloc (the decode layer without a
workspace argument, on the library's own scratch array): its outputs equal
moe_decode_layer's bit for bit, on two calls in a row, the second with a
smaller input (fewer tokens, another layer shape), and sizes beyond the
scratch are refused."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from parity import GpuLayer, need_gpu

pytestmark = pytest.mark.gpu


def _outputs(T, k, d, dev):
    return dict(idx=torch.empty((T, k), dtype=torch.int32, device=dev),
                w=torch.empty((T, k), dtype=torch.float32, device=dev),
                slot=torch.empty((T, k), dtype=torch.int32, device=dev),
                miss_expert=torch.full((T * k,), -1, dtype=torch.int32, device=dev),
                miss_pair=torch.full((T * k,), -1, dtype=torch.int32, device=dev),
                n_miss=torch.zeros((4,), dtype=torch.int32, device=dev),
                y=torch.empty((T, d), dtype=torch.float32, device=dev))


def test_noalloc_equals_decode_layer_twice():
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    cases = [
        # the model's layer at T = 4 (the larger call), then a smaller one
        (synth.config_shape(1), synth.FMT_Q2SM, 4, 0.8),
        (synth.LayerShape(100, 5, 256, 128, True), synth.FMT_Q3G, 2, 0.6),
    ]
    for n, (shape, fmt, T, frac) in enumerate(cases):
        E, k, d = shape.n_experts, shape.top_k, shape.d_model
        rng = np.random.default_rng(40 + n)
        resident = np.sort(rng.choice(E, int(frac * E), replace=False))
        x = synth.make_x(5, n, T, d).to(dev)
        logits = synth.make_logits(5, n, T, E, 1.5).to(dev)
        chosen = set(np.argsort(-logits.cpu().numpy(), axis=1, kind="stable")[:, :k]
                     .reshape(-1).tolist())
        L = GpuLayer(5, n, shape, fmt, dev, resident=resident, only_experts=chosen)
        tab = L.table_dev(dev)
        ref = _outputs(T, k, d, dev)
        bf.decode_layer(L.layer_obj, x, logits, tab, **ref)
        got = _outputs(T, k, d, dev)
        bf.decode_layer_noalloc(L.layer_obj, x, logits, tab, **got)
        torch.cuda.synchronize()
        for key in ref:
            assert torch.equal(got[key], ref[key]), (n, key)
        assert int(ref["n_miss"][1]) > 0 or frac == 1.0


def test_noalloc_refuses_sizes_beyond_the_scratch():
    import bit_expert_ffn_top_amd as bf
    from bit_expert_ffn_top_amd import _binding as b
    dev = need_gpu()
    # d_model 2048, d_ff 4096, top-16, T = 4: 4 * 17 * 128 * 2048 * 4 bytes of partials
    d, f, E, k, T = 2048, 4096, 64, 16, 4
    sb = synth.slot_bytes(synth.FMT_Q2SM, d, f)
    pool = torch.zeros((1, sb), dtype=torch.uint8, device=dev)
    L = b.MoeLayerC(d, f, E, k, synth.FMT_Q2SM, 1, -1, 0, sb, pool.data_ptr())
    assert b.lib().moe_decode_workspace_bytes(ctypes.byref(L), T) > (16 << 20)
    buf = torch.zeros((1 << 16,), dtype=torch.float32, device=dev)
    p = ctypes.c_void_p(buf.data_ptr())
    q = ctypes.c_void_p(buf.data_ptr() + 4096)
    st = b.lib().moe_decode_layer_noalloc(ctypes.byref(L), p, T, p, p, p, p, p, p, None, p, q,
                                          None)
    assert st == b.MOE_ENOSPC
