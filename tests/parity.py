"""Shared helpers of the GPU parity tests (not a test module)."""
import numpy as np
import pytest
import torch

import oracle
import synth

# fp32 outputs: max|err| <= 2e-3 * max|ref| and sum|err| / sum|ref| <= 1e-4,
# on the layer output y and on its update y - x.
MAX_REL = 2e-3
MEAN_REL = 1e-4


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def check_close(got, ref, x=None, what="y", max_rel=MAX_REL, mean_rel=MEAN_REL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    pairs = [(what, got, ref)]
    if x is not None:
        x = np.asarray(x, dtype=np.float64)
        pairs.append((what + "-x", got - x, ref - x))
    for name, g, r in pairs:
        err = np.abs(g - r)
        scale = np.abs(r).max()
        if scale == 0:
            assert err.max() == 0, f"{name}: expected zeros, max err {err.max()}"
            continue
        assert err.max() <= max_rel * scale, f"{name}: max err {err.max():.3e} > {max_rel}*{scale:.3e}"
        mr = err.sum() / np.abs(r).sum()
        assert mr <= mean_rel, f"{name}: mean relative error {mr:.3e} > {mean_rel}"


class GpuLayer:
    """A layer's packed pool on the device plus the oracle's view of it."""

    def __init__(self, cfg, layer, shape, fmt, dev, resident=None, shared=True, seed_slots=True,
                 only_experts=None):
        self.cfg, self.layer, self.shape, self.fmt = cfg, layer, shape, fmt
        E = shape.n_experts
        self.E = E
        resident = np.arange(E) if resident is None else np.asarray(resident)
        ids = [int(e) for e in resident] + ([E] if shared else [])
        rng = np.random.default_rng(1000 + 7 * layer + cfg)
        order = rng.permutation(len(ids)) if seed_slots else np.arange(len(ids))
        self.slot_expert = [0] * len(ids)
        for i, s in enumerate(order):
            self.slot_expert[int(s)] = ids[i]
        self.table = np.full(E, -1, dtype=np.int32)
        self.shared_slot = -1
        for s, e in enumerate(self.slot_expert):
            if e == E:
                self.shared_slot = s
            else:
                self.table[e] = s
        sb = synth.slot_bytes(fmt, shape.d_model, shape.d_ff)
        self.pool = torch.zeros((len(ids), sb), dtype=torch.uint8, device=dev)
        want = set(ids) if only_experts is None else set(only_experts) | ({E} if shared else set())
        fill = [s for s, e in enumerate(self.slot_expert) if e in want]
        self._bytes = {}
        if fill:
            experts = [self.slot_expert[s] for s in fill]
            packed = synth.make_layer_pool(cfg, layer, experts, device=dev, fmt=fmt, shape=shape)
            self.pool[fill] = packed
            host = packed.cpu().numpy()
            for j, s in enumerate(fill):
                self._bytes[s] = host[j]
        self._w = {}
        import bit_expert_ffn_top_amd as bf
        self.layer_obj = bf.MoeLayer(shape.d_model, shape.d_ff, E, shape.top_k, fmt, self.pool,
                                     self.shared_slot)

    def weights_of_slot(self, s):
        if s not in self._w:
            self._w[s] = oracle.unpack_expert(self._bytes[s], self.fmt, self.shape.d_model,
                                              self.shape.d_ff)
        return self._w[s]

    def weights_of_expert(self, e):
        s = self.shared_slot if e == self.E else int(self.table[e])
        return self.weights_of_slot(s)

    def table_dev(self, dev):
        return torch.tensor(self.table, dtype=torch.int32, device=dev)


class HostTier:
    """Every expert of a layer in pinned host memory at a permuted slot
    order (only the experts in `fill` are generated; the other slots hold
    zeros and must never be read for a nonzero term)."""

    def __init__(self, cfg, layer, shape, fmt, fill, absent=(), device_pool=False, seed=0):
        import bit_expert_ffn_top_amd as bf
        E = shape.n_experts
        rng = np.random.default_rng(500 + seed)
        order = rng.permutation(E)                  # host slot h holds expert order[h]
        self.host_slot = np.empty(E, np.int32)
        self.host_slot[order] = np.arange(E, dtype=np.int32)
        for e in absent:
            self.host_slot[e] = -1
        self.fmt, self.shape = fmt, shape
        sb = synth.slot_bytes(fmt, shape.d_model, shape.d_ff)
        if device_pool:
            self.pool = torch.zeros((E, sb), dtype=torch.uint8, device="cuda:0")
        else:
            self.pool = torch.zeros((E, sb), dtype=torch.uint8, pin_memory=True)
        fill = sorted(set(int(e) for e in fill) - set(absent))
        self._bytes = {}
        if fill:
            packed = synth.make_layer_pool(cfg, layer, fill, device="cuda:0", fmt=fmt,
                                           shape=shape).cpu()
            for j, e in enumerate(fill):
                h = int(self.host_slot[e])
                self.pool[h] = packed[j].to(self.pool.device)
                self._bytes[h] = packed[j].numpy()
        self._w = {}
        self.tier = bf.HostTier(shape.d_model, shape.d_ff, E, shape.top_k, fmt, self.pool)

    def weights_of_host_slot(self, h):
        if h not in self._w:
            self._w[h] = oracle.unpack_expert(self._bytes[h], self.fmt, self.shape.d_model,
                                              self.shape.d_ff)
        return self._w[h]

    def table_dev(self):
        return torch.tensor(self.host_slot, dtype=torch.int32, device="cuda:0")
