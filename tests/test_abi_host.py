"""C ABI checks that need no GPU: the library loads, exports every function
the header declares, computes slot sizes like the two independent layout
implementations, and rejects bad arguments on the host before any HIP call
(so these calls never touch a device)."""
import ctypes
import os
import re

import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitffn_moe.h")

bf = pytest.importorskip("bit_expert_ffn_top_amd")


def _lib():
    try:
        return bf.lib()
    except RuntimeError as e:
        pytest.skip(str(e))


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\*?\s+\*?(moe_\w+)\s*\(", text, flags=re.M)))


def test_header_symbols_exported():
    lib = _lib()
    names = _declared_functions()
    assert len(names) >= 12, names
    for n in names:
        assert hasattr(lib, n), n
    from bit_expert_ffn_top_amd import _binding
    assert set(names) == set(_binding.SIGNATURES), set(names) ^ set(_binding.SIGNATURES)


def test_version_and_status_strings():
    lib = _lib()
    assert lib.moe_abi_version() == 1
    for st in (0, -1, -2, -3, -4, -5):
        assert lib.moe_status_str(st)
    assert lib.moe_status_str(-99) == b"unknown status"


@pytest.mark.parametrize("fmt", [1, 2, 3])
@pytest.mark.parametrize("d,f", [(64, 32), (256, 128), (2048, 768), (512, 96), (1024, 2048),
                                 (192, 160)])
def test_slot_bytes_matches_layouts(fmt, d, f):
    lib = _lib()
    got = lib.moe_slot_bytes(fmt, d, f)
    assert got == synth.slot_bytes(fmt, d, f) == oracle.slot_size(fmt, d, f)


def test_slot_bytes_rejects():
    lib = _lib()
    assert lib.moe_slot_bytes(4, 256, 128) == -3
    assert lib.moe_slot_bytes(2, 96, 128) == -1       # d not a multiple of 64
    assert lib.moe_slot_bytes(2, 4096, 128) == -1     # d too large
    assert lib.moe_slot_bytes(2, 256, 80) == -1       # d_ff not a multiple of 32
    assert lib.moe_slot_bytes(2, 256, 8192) == -1     # d_ff too large


FAKE = 0x7F0000000000  # never dereferenced: every call below fails its host checks


def _p(off=0):
    return ctypes.c_void_p(FAKE + off)


def test_route_topk_host_checks():
    lib = _lib()
    s = ctypes.c_void_p(0)
    assert lib.moe_route_topk(_p(), 1, 0, 1, _p(), _p(), s) == -1          # E = 0
    assert lib.moe_route_topk(_p(), 1, 2000, 4, _p(), _p(), s) == -1       # E > 1024
    assert lib.moe_route_topk(_p(), 1, 64, 65, _p(), _p(), s) == -1        # k > 64
    assert lib.moe_route_topk(_p(), 1, 8, 9, _p(), _p(), s) == -1          # k > E
    assert lib.moe_route_topk(_p(), -1, 64, 4, _p(), _p(), s) == -1
    assert lib.moe_route_topk(None, 1, 64, 4, _p(), _p(), s) == -1
    assert lib.moe_route_topk(_p(4), 1, 64, 4, _p(), _p(), s) == -2        # misaligned
    assert lib.moe_route_topk(None, 0, 64, 4, None, None, s) == 0          # T = 0: no-op


def test_router_logits_host_checks():
    lib = _lib()
    s = ctypes.c_void_p(0)
    call = lambda T=1, d=2048, E=512, x=_p(), w=_p(1 << 20), out=_p(1 << 24): \
        lib.moe_router_logits(x, T, d, w, E, out, s)
    assert call(T=0) == -1
    assert call(T=5) == -1                                      # decode / verify only
    assert call(d=96) == -1                                     # not a multiple of 64
    assert call(d=4096) == -1
    assert call(E=0) == -1
    assert call(E=2000) == -1
    assert call(x=None) == -1
    assert call(w=None) == -1
    assert call(out=None) == -1
    assert call(out=_p()) == -1                                 # logits alias x
    assert call(out=_p(1 << 20)) == -1                          # logits alias w
    assert call(x=_p(4)) == -2
    assert call(w=_p((1 << 20) + 8)) == -2
    assert call(out=_p((1 << 24) + 4)) == -2


def test_lookup_host_checks():
    lib = _lib()
    s = ctypes.c_void_p(0)
    assert lib.moe_cache_lookup(_p(), 1, 0, _p(), 64, _p(), _p(), _p(), _p(), None, 0, s) == -1
    assert lib.moe_cache_lookup(None, 1, 4, _p(), 64, _p(), _p(), _p(), _p(), None, 0, s) == -1
    assert lib.moe_cache_lookup(_p(8), 1, 4, _p(), 64, _p(), _p(), _p(), _p(), None, 0, s) == -2
    # large inputs need a workspace
    need = lib.moe_lookup_workspace_bytes(8192, 10, 512)
    assert need > 0 and lib.moe_lookup_workspace_bytes(4, 10, 512) == 0
    assert lib.moe_cache_lookup(_p(), 8192, 10, _p(), 512, _p(), _p(), _p(), _p(), None, 0, s) == -1
    assert lib.moe_cache_lookup(_p(), 8192, 10, _p(), 512, _p(), _p(), _p(), _p(), _p(),
                                need - 1, s) == -4


def _layer(**kw):
    v = dict(d_model=2048, d_ff=768, n_experts=512, top_k=10, fmt=2, n_slots=513,
             shared_slot=512, reserved=0, slot_bytes=synth.slot_bytes(2, 2048, 768), pool=FAKE)
    v.update(kw)
    from bit_expert_ffn_top_amd._binding import MoeLayerC
    return MoeLayerC(**v)


def test_decode_host_checks():
    lib = _lib()
    s = ctypes.c_void_p(0)
    L = _layer()
    need = lib.moe_decode_workspace_bytes(ctypes.byref(L), 1)
    assert need > 0
    args = lambda L, T=1, ws=need, y=_p(1 << 20): (ctypes.byref(L), _p(), T, _p(), _p(), _p(), y, _p(), ws, s)
    assert lib.moe_expert_ffn_decode(*args(L, ws=need - 1)) == -4
    assert lib.moe_expert_ffn_decode(*args(L, T=5)) == -1
    assert lib.moe_expert_ffn_decode(*args(_layer(top_k=20), T=4)) == -1   # T*k > 64
    assert lib.moe_expert_ffn_decode(*args(L, y=_p())) == -1               # y aliases x
    assert lib.moe_expert_ffn_decode(*args(_layer(fmt=7))) == -3
    assert lib.moe_expert_ffn_decode(*args(_layer(slot_bytes=12345))) == -3
    assert lib.moe_expert_ffn_decode(*args(_layer(pool=FAKE + 16))) == -2
    assert lib.moe_expert_ffn_decode(*args(_layer(shared_slot=513))) == -1
    assert lib.moe_expert_ffn_decode(*args(_layer(reserved=1))) == -1
    assert lib.moe_expert_ffn_decode(*args(_layer(top_k=0))) == -1
    assert lib.moe_expert_ffn_decode(*args(_layer(d_model=3000))) == -1
    assert lib.moe_decode_workspace_bytes(ctypes.byref(L), 5) == 0


def test_prefill_host_checks():
    lib = _lib()
    s = ctypes.c_void_p(0)
    L = _layer()
    need = lib.moe_prefill_workspace_bytes(ctypes.byref(L), 8192)
    assert need > 0
    def call(L, T=8192, ws=need, shared=_p()):
        return lib.moe_expert_ffn_prefill(ctypes.byref(L), _p(), T, _p(), _p(), _p(), _p(), _p(),
                                          shared, _p(), ws, s)
    assert call(L, ws=need - 1) == -4
    assert call(L, T=0) == -1
    assert call(L, T=70000) == -1
    assert call(_layer(shared_slot=-1)) == -1                               # shared out, no shared
    L64 = _layer(d_model=64, slot_bytes=synth.slot_bytes(2, 64, 768))
    assert call(L64, ws=1 << 40) == -1                                      # d not a multiple of 128
    big = _layer(top_k=64, d_ff=4096, slot_bytes=synth.slot_bytes(2, 2048, 4096))
    assert call(big, T=65536, ws=1 << 40) == -1                            # h past 4 GiB


def test_combine_host_checks():
    lib = _lib()
    s = ctypes.c_void_p(0)
    assert lib.moe_combine(_p(), 3, 1, 64, 4, _p(), _p(), _p(), None, _p(), s) == -1
    assert lib.moe_combine(_p(), 0, 1, 66, 4, _p(), _p(), _p(), None, _p(), s) == -1
    assert lib.moe_combine(_p(), 0, 1, 64, 4, None, _p(), _p(), None, _p(), s) == -1
    assert lib.moe_combine(_p(), 1, 1, 64, 4, _p(), _p(), _p(), None, _p(), s) == -1   # bf16 alias
    assert lib.moe_combine(_p(4), 0, 1, 64, 4, _p(), _p(), _p(), None, _p(1 << 12), s) == -2
    assert lib.moe_combine(None, 0, 0, 64, 4, None, None, None, None, None, s) == 0


def test_decode_misses_host_checks():
    lib = _lib()
    s = ctypes.c_void_p(0)
    H = _layer(shared_slot=-1, n_slots=512)
    need = lib.moe_decode_workspace_bytes(ctypes.byref(H), 1)
    def call(H, T=1, max_rank=10, ws=need, y=_p(1 << 20)):
        return lib.moe_decode_misses(ctypes.byref(H), _p(), T, _p(), _p(), _p(), _p(), max_rank,
                                     y, _p(), ws, s)
    assert call(_layer(shared_slot=3, n_slots=512)) == -1                   # shared slot in the tier
    assert call(H, max_rank=11) == -1
    assert call(H, max_rank=-1) == -1
    assert call(H, T=5) == -1
    assert call(H, ws=need - 1) == -4
    assert call(H, y=_p()) == -1                                            # y aliases x
    assert call(_layer(shared_slot=-1, fmt=9)) == -3

    def phases(ph, x=_p(), y=_p(1 << 20), w=_p(1 << 21)):
        return lib.moe_decode_misses_phases(ctypes.byref(H), x, 1, _p(), _p(), w, _p(), 10, y,
                                            _p(), need, ph, s)
    assert phases(0) == -1
    assert phases(4) == -1
    assert phases(1, x=None) == -1                                           # the read needs x
    assert phases(2, y=None) == -1                                           # the join needs y ...
    assert phases(2, w=None) == -1                                           # ... and w
    assert phases(3, y=_p()) == -1                                           # y aliases x
    assert phases(2, x=None, y=_p(8)) == -2


def test_decode_layer_tiers_host_checks():
    lib = _lib()
    s = ctypes.c_void_p(0)
    L = _layer()
    H = _layer(shared_slot=-1, n_slots=512)
    need = lib.moe_decode_workspace_bytes(ctypes.byref(L), 1)
    def call(L=L, H=H, T=1, max_rank=10, ws=need, wsp=_p(), y=_p(1 << 20), host=_p(1 << 24)):
        return lib.moe_decode_layer_tiers(ctypes.byref(L), ctypes.byref(H), host, max_rank, _p(),
                                          T, _p(1 << 16), _p(1 << 17), _p(1 << 18), _p(1 << 19),
                                          _p(1 << 21), _p(1 << 22), None, _p(1 << 23), y, wsp,
                                          ws, s)
    assert call(ws=need - 1) == -4
    assert call(wsp=None) == -1
    assert call(wsp=_p(16)) == -2
    assert call(host=None) == -1
    assert call(host=_p(4)) == -2
    assert call(max_rank=11) == -1
    assert call(max_rank=-1) == -1
    assert call(T=5) == -1
    assert call(y=_p()) == -1                                                # y aliases x
    assert call(H=_layer(shared_slot=3, n_slots=512)) == -1                  # shared slot in the tier
    assert call(H=_layer(shared_slot=-1, n_slots=512, top_k=8)) == -1        # other top_k
    assert call(H=_layer(shared_slot=-1, n_slots=512, n_experts=256)) == -1  # other E
    assert call(H=_layer(shared_slot=-1, n_slots=512, fmt=3,
                         slot_bytes=synth.slot_bytes(3, 2048, 768))) == -1   # other format
    assert call(H=_layer(shared_slot=-1, n_slots=512, pool=FAKE + 16)) == -2
    assert call(L=_layer(fmt=9)) == -3


def test_cache_policy_host_checks():
    lib = _lib()
    s = ctypes.c_void_p(0)
    assert lib.moe_cache_count(_p(), 10, 0, _p(), s) == -1
    assert lib.moe_cache_count(_p(), 10, 2000, _p(), s) == -1
    assert lib.moe_cache_count(_p(), -1, 512, _p(), s) == -1
    assert lib.moe_cache_count(None, 0, 512, None, s) == 0                  # nothing to count
    assert lib.moe_cache_count(_p(4), 10, 512, _p(), s) == -2

    def plan(E=512, n_slots=95, shared=94, max_swaps=8, shift=1, **kw):
        a = dict(counts=_p(), soe=_p(), eos=_p(), hs=_p(), swaps=_p(), n=_p())
        a.update(kw)
        return lib.moe_cache_plan(a["counts"], E, a["soe"], a["eos"], n_slots, shared, a["hs"],
                                  512, max_swaps, shift, a["swaps"], a["n"], s)
    assert plan(E=0) == -1
    assert plan(n_slots=0) == -1
    assert plan(n_slots=5000) == -1
    assert plan(shared=95) == -1
    assert plan(max_swaps=0) == -1
    assert plan(max_swaps=1025) == -1
    assert plan(shift=32) == -1
    assert plan(hs=None) == -1
    assert plan(swaps=_p(8)) == -2

    L = _layer()
    H = _layer(n_slots=512, shared_slot=-1)
    fill = lambda L, H, m=8, sw=_p(): lib.moe_cache_fill(ctypes.byref(L), ctypes.byref(H), sw, _p(),
                                                         m, s)
    assert fill(L, _layer(fmt=1, slot_bytes=synth.slot_bytes(1, 2048, 768))) == -3
    assert fill(L, H, m=0) == -1
    assert fill(L, H, sw=_p(4)) == -2
    assert fill(L, _layer(pool=FAKE + 16)) == -2
    assert lib.moe_cache_commit(_p(), 0, _p(), _p(), 8, s) == -1
    assert lib.moe_cache_commit(_p(), 512, _p(), _p(), 0, s) == -1
    assert lib.moe_cache_commit(_p(), 512, None, _p(), 8, s) == -1


def test_stage_layer_host_checks():
    lib = _lib()
    s = ctypes.c_void_p(0)
    import numpy as np
    E = 512
    C = _layer(n_slots=95, shared_slot=94)
    H = _layer(n_slots=512, shared_slot=-1)
    soe = np.full(E, -1, np.int32)
    soe[:94] = np.arange(94)
    hs = np.arange(E, dtype=np.int32)
    sb = synth.slot_bytes(2, 2048, 768)
    def call(C=C, H=H, soe=soe, hs=hs, nbytes=(E + 1) * sb, st=_p()):
        return lib.moe_stage_layer(ctypes.byref(C), soe.ctypes.data, ctypes.byref(H),
                                   hs.ctypes.data, st, nbytes, s)
    assert call(nbytes=E * sb) == -4
    assert call(st=_p(16)) == -2
    assert call(H=_layer(n_slots=512, shared_slot=-1, n_experts=500)) == -1
    assert call(H=_layer(fmt=1, slot_bytes=synth.slot_bytes(1, 2048, 768))) == -3
    bad = hs.copy()
    bad[200] = -1                                     # expert 200: neither tier
    assert call(hs=bad) == -1
    bad = hs.copy()
    bad[200] = 512                                    # host slot out of range
    assert call(hs=bad) == -1
    bad = soe.copy()
    bad[300] = 94                                     # the shared slot is no expert's home
    assert call(soe=bad, hs=np.where(np.arange(E) == 300, -1, hs).astype(np.int32)) == -1


def test_decode_stack_host_checks():
    lib = _lib()
    s = ctypes.c_void_p(0)
    from bit_expert_ffn_top_amd._binding import MoeStackLayerC
    sb = synth.slot_bytes(2, 2048, 768)

    def layer(**kw):
        v = dict(pool=FAKE, slot_bytes=sb, n_slots=513, fmt=2, shared_slot=512, reserved=0,
                 slot_of_expert=_p(1 << 16), logits=_p(1 << 17), addend=None, y=_p(1 << 18),
                 idx=None, w=None, slot=None, miss_expert=None, miss_pair=None, n_miss=None)
        v.update(kw)
        return MoeStackLayerC(**v)

    need = lib.moe_decode_stack_workspace_bytes(2048, 768, 512, 10, 1)
    assert need > 0
    assert lib.moe_decode_stack_workspace_bytes(2048, 768, 512, 10, 5) == 0
    assert lib.moe_decode_stack_workspace_bytes(2048, 768, 512, 20, 4) == 0   # T*k > 64
    assert lib.moe_decode_stack_workspace_bytes(2048, 768, 1025, 10, 1) == 0

    def call(layers, n=None, T=1, k=10, E=512, d=2048, f=768, x=_p(1 << 21), ws=_p(1 << 22),
             nb=need):
        arr = (MoeStackLayerC * len(layers))(*layers)
        return lib.moe_decode_stack(d, f, E, k, T, len(layers) if n is None else n, arr, x, ws,
                                    nb, s)

    ok = [layer(y=None), layer()]
    assert call(ok, n=0) == -1
    assert call(ok, T=5) == -1
    assert call(ok, T=4, k=20) == -1
    assert call(ok, nb=need - 1) == -4
    assert call(ok, ws=_p((1 << 22) + 16)) == -2                      # workspace 256-aligned
    assert call(ok, x=None) == -1
    assert call([layer(), layer(y=None)]) == -1                        # last y required
    assert call([layer(y=None), layer(fmt=7)]) == -3
    assert call([layer(y=None), layer(slot_bytes=sb + 256)]) == -3
    assert call([layer(y=None), layer(reserved=1)]) == -1
    assert call([layer(y=None), layer(shared_slot=513)]) == -1
    assert call([layer(y=None), layer(logits=None)]) == -1
    assert call([layer(y=None), layer(idx=_p(1 << 19))]) == -1         # routing: all or none
    assert call([layer(y=None), layer(n_miss=_p(1 << 19))]) == -1      # with miss_expert only
    assert call([layer(y=None), layer(pool=FAKE + 16)]) == -2
    assert call([layer(y=None), layer(addend=_p((1 << 19) + 4))]) == -2
    assert call([layer(y=None), layer(y=_p(1 << 21))]) == -1           # y aliases x
