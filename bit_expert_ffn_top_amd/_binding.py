"""ctypes binding of libbitffn_moe.so (include/bitffn_moe.h).

Argument marshalling only: tensors are checked for device, dtype and shape,
their data pointers and the current HIP stream are passed to the C ABI, and
any output tensor the caller did not supply is allocated with torch.  Every
step of the computation runs in the library's kernels.  There is no fallback:
if the library cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

LIB_NAME = "libbitffn_moe.so"
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

MOE_OK, MOE_EINVAL, MOE_EALIGN, MOE_EFORMAT, MOE_ENOSPC, MOE_EHIP = 0, -1, -2, -3, -4, -5
FMT_Q2S, FMT_Q2SM, FMT_Q3G = 1, 2, 3
DTYPE_F32, DTYPE_BF16 = 0, 1

# every symbol the header declares, with its ctypes signature
_c_int, _c_i64, _c_sz, _vp = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p


class MoeLayerC(ctypes.Structure):
    _fields_ = [
        ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
        ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("fmt", ctypes.c_int32), ("n_slots", ctypes.c_int32),
        ("shared_slot", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("slot_bytes", ctypes.c_int64), ("pool", ctypes.c_void_p),
    ]


class MoeStackLayerC(ctypes.Structure):
    _fields_ = [
        ("pool", ctypes.c_void_p), ("slot_bytes", ctypes.c_int64),
        ("n_slots", ctypes.c_int32), ("fmt", ctypes.c_int32),
        ("shared_slot", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("slot_of_expert", ctypes.c_void_p), ("logits", ctypes.c_void_p),
        ("addend", ctypes.c_void_p), ("y", ctypes.c_void_p),
        ("idx", ctypes.c_void_p), ("w", ctypes.c_void_p), ("slot", ctypes.c_void_p),
        ("miss_expert", ctypes.c_void_p), ("miss_pair", ctypes.c_void_p),
        ("n_miss", ctypes.c_void_p),
    ]


_LP = ctypes.POINTER(MoeLayerC)
_SLP = ctypes.POINTER(MoeStackLayerC)
SIGNATURES = {
    "moe_abi_version": (_c_int, []),
    "moe_status_str": (ctypes.c_char_p, [_c_int]),
    "moe_last_hip_error": (_c_int, []),
    "moe_slot_bytes": (_c_i64, [_c_int, _c_int, _c_int]),
    "moe_router_logits": (_c_int, [_vp, _c_int, _c_int, _vp, _c_int, _vp, _vp]),
    "moe_route_topk": (_c_int, [_vp, _c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "moe_lookup_workspace_bytes": (_c_sz, [_c_int, _c_int, _c_int]),
    "moe_cache_lookup": (_c_int, [_vp, _c_int, _c_int, _vp, _c_int, _vp, _vp, _vp, _vp, _vp,
                                  _c_sz, _vp]),
    "moe_decode_workspace_bytes": (_c_sz, [_LP, _c_int]),
    "moe_expert_ffn_decode": (_c_int, [_LP, _vp, _c_int, _vp, _vp, _vp, _vp, _vp, _c_sz, _vp]),
    "moe_decode_layer": (_c_int, [_LP, _vp, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _vp, _c_sz, _vp]),
    "moe_decode_layer_noalloc": (_c_int, [_LP, _vp, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                          _vp, _vp, _vp]),
    "moe_decode_stack_workspace_bytes": (_c_sz, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "moe_decode_stack": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _SLP, _vp,
                                  _vp, _c_sz, _vp]),
    "moe_decode_misses": (_c_int, [_LP, _vp, _c_int, _vp, _vp, _vp, _vp, _c_int, _vp, _vp,
                                   _c_sz, _vp]),
    "moe_decode_misses_phases": (_c_int, [_LP, _vp, _c_int, _vp, _vp, _vp, _vp, _c_int, _vp,
                                          _vp, _c_sz, _c_int, _vp]),
    "moe_decode_layer_tiers": (_c_int, [_LP, _LP, _vp, _c_int, _vp, _c_int, _vp, _vp, _vp, _vp,
                                        _vp, _vp, _vp, _vp, _vp, _vp, _c_sz, _vp]),
    "moe_cache_count": (_c_int, [_vp, _c_int, _c_int, _vp, _vp]),
    "moe_cache_plan": (_c_int, [_vp, _c_int, _vp, _vp, _c_int, _c_int, _vp, _c_int, _c_int,
                                _c_int, _vp, _vp, _vp]),
    "moe_cache_fill": (_c_int, [_LP, _LP, _vp, _vp, _c_int, _vp]),
    "moe_cache_commit": (_c_int, [_vp, _c_int, _vp, _vp, _c_int, _vp]),
    "moe_stage_layer": (_c_int, [_LP, _vp, _LP, _vp, _vp, _c_sz, _vp]),
    "moe_prefill_workspace_bytes": (_c_sz, [_LP, _c_int]),
    "moe_expert_ffn_prefill": (_c_int, [_LP, _vp, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _c_sz, _vp]),
    "moe_combine": (_c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp]),
}

_lib = None


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{LIB_NAME} is not built; run `python -m bit_expert_ffn_top_amd.build`")
        handle = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = lib().moe_status_str(status).decode()
        if status == MOE_EHIP:
            msg += f" (hip error {lib().moe_last_hip_error()})"
        super().__init__(f"{what}: {msg} [{status}]")
        self.status = status


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoeError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, dtype, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _shape(t: torch.Tensor, shape, name: str):
    """t must have exactly this shape (None: any extent).  Checked before the
    device checks, so that a wrong size is reported as such."""
    if t.dim() != len(shape) or any(s is not None and a != s for a, s in zip(t.shape, shape)):
        parts = ["*" if s is None else str(s) for s in shape]
        want = "(" + ", ".join(parts) + ("," if len(parts) == 1 else "") + ")"
        raise ValueError(f"{name}: shape {want} expected, got {tuple(t.shape)}")
    return t


def _at_least(t: torch.Tensor, n: int, name: str):
    if t.numel() < n:
        raise ValueError(f"{name}: at least {n} elements expected, got {t.numel()}")
    return t


@dataclasses.dataclass
class MoeLayer:
    """One layer's packed expert pool in device memory."""
    d_model: int
    d_ff: int
    n_experts: int
    top_k: int
    fmt: int
    pool: torch.Tensor            # uint8 [n_slots, slot_bytes] on the device
    shared_slot: int = -1

    def c_struct(self) -> MoeLayerC:
        _dev(self.pool, torch.uint8, "pool")
        n_slots, sb = self.pool.shape
        return MoeLayerC(self.d_model, self.d_ff, self.n_experts, self.top_k, self.fmt,
                         n_slots, self.shared_slot, 0, sb, self.pool.data_ptr())


def abi_version() -> int:
    return lib().moe_abi_version()


def slot_bytes(fmt: int, d_model: int, d_ff: int) -> int:
    v = lib().moe_slot_bytes(fmt, d_model, d_ff)
    _check(int(v) if v < 0 else 0, "moe_slot_bytes")
    return int(v)


def router_logits(x: torch.Tensor, w: torch.Tensor, logits=None, stream=None):
    """logits [T, E] = x [T, d] (fp32) times the bf16 router weights w [E, d]."""
    _dev(_shape(x, (None, None), "x"), torch.float32, "x")
    T, d = x.shape
    _dev(_shape(w, (None, d), "w"), torch.bfloat16, "w")
    E = w.shape[0]
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _dev(_shape(logits, (T, E), "logits"), torch.float32, "logits")
    _check(lib().moe_router_logits(_ptr(x), T, d, _ptr(w), E, _ptr(logits), _stream(stream)),
           "moe_router_logits")
    return logits


def route_topk(logits: torch.Tensor, k: int, idx=None, w=None, stream=None):
    _shape(logits, (None, None), "logits")
    _dev(logits, torch.float32, "logits")
    T, E = logits.shape
    if idx is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _dev(_shape(idx, (T, k), "idx"), torch.int32, "idx")
    _dev(_shape(w, (T, k), "w"), torch.float32, "w")
    _check(lib().moe_route_topk(_ptr(logits), T, E, k, _ptr(idx), _ptr(w), _stream(stream)),
           "moe_route_topk")
    return idx, w


def lookup_workspace_bytes(T: int, k: int, E: int) -> int:
    return int(lib().moe_lookup_workspace_bytes(T, k, E))


def cache_lookup(idx: torch.Tensor, slot_of_expert: torch.Tensor, slot=None, miss_expert=None,
                 miss_pair=None, n_miss=None, ws=None, want_pairs=True, stream=None):
    _shape(idx, (None, None), "idx")
    _shape(slot_of_expert, (None,), "slot_of_expert")
    _dev(idx, torch.int32, "idx")
    _dev(slot_of_expert, torch.int32, "slot_of_expert")
    T, k = idx.shape
    E = slot_of_expert.shape[0]
    dev = idx.device
    n = T * k
    slot = torch.empty((T, k), dtype=torch.int32, device=dev) if slot is None else slot
    miss_expert = torch.full((max(n, 1),), -1, dtype=torch.int32, device=dev) if miss_expert is None else miss_expert
    if want_pairs and miss_pair is None:
        miss_pair = torch.full((max(n, 1),), -1, dtype=torch.int32, device=dev)
    n_miss = torch.zeros((4,), dtype=torch.int32, device=dev) if n_miss is None else n_miss
    _dev(_shape(slot, (T, k), "slot"), torch.int32, "slot")
    _dev(_at_least(miss_expert, n, "miss_expert"), torch.int32, "miss_expert")
    if miss_pair is not None:
        _dev(_at_least(miss_pair, n, "miss_pair"), torch.int32, "miss_pair")
    _dev(_at_least(n_miss, 2, "n_miss"), torch.int32, "n_miss")
    need = lookup_workspace_bytes(T, k, E)
    if need and ws is None:
        ws = torch.empty((need,), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().moe_cache_lookup(_ptr(idx), T, k, _ptr(slot_of_expert), E, _ptr(slot),
                                  _ptr(miss_expert), _ptr(miss_pair), _ptr(n_miss), _ptr(ws),
                                  ws_bytes, _stream(stream)), "moe_cache_lookup")
    return slot, miss_expert, miss_pair, n_miss


def decode_workspace_bytes(layer: MoeLayer, T: int) -> int:
    L = layer.c_struct()
    return int(lib().moe_decode_workspace_bytes(ctypes.byref(L), T))


def expert_ffn_decode(layer: MoeLayer, x, idx, slot, w, y=None, ws=None, stream=None):
    _dev(_shape(x, (None, layer.d_model), "x"), torch.float32, "x")
    T = x.shape[0]
    for name, t, dt in (("idx", idx, torch.int32), ("slot", slot, torch.int32),
                        ("w", w, torch.float32)):
        _dev(_shape(t, (T, layer.top_k), name), dt, name)
    L = layer.c_struct()
    if y is None:
        y = torch.empty_like(x)
    _dev(_shape(y, tuple(x.shape), "y"), torch.float32, "y")
    if ws is None:
        ws = torch.empty((decode_workspace_bytes(layer, T),), dtype=torch.uint8, device=x.device)
    _check(lib().moe_expert_ffn_decode(ctypes.byref(L), _ptr(x), T, _ptr(idx), _ptr(slot),
                                       _ptr(w), _ptr(y), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_expert_ffn_decode")
    return y


def decode_layer(layer: MoeLayer, x, logits, slot_of_expert, idx=None, w=None, slot=None,
                 miss_expert=None, miss_pair=None, n_miss=None, y=None, ws=None,
                 want_pairs=True, stream=None):
    """Route, look up and run one decode layer (moe_decode_layer).
    Returns (y, idx, w, slot, miss_expert, miss_pair, n_miss)."""
    _dev(_shape(x, (None, layer.d_model), "x"), torch.float32, "x")
    T = x.shape[0]
    k = layer.top_k
    _dev(_shape(logits, (T, layer.n_experts), "logits"), torch.float32, "logits")
    _dev(_shape(slot_of_expert, (layer.n_experts,), "slot_of_expert"), torch.int32,
         "slot_of_expert")
    dev = x.device
    n = T * k
    idx = torch.empty((T, k), dtype=torch.int32, device=dev) if idx is None else idx
    w = torch.empty((T, k), dtype=torch.float32, device=dev) if w is None else w
    slot = torch.empty((T, k), dtype=torch.int32, device=dev) if slot is None else slot
    if miss_expert is None:
        miss_expert = torch.full((n,), -1, dtype=torch.int32, device=dev)
    if want_pairs and miss_pair is None:
        miss_pair = torch.full((n,), -1, dtype=torch.int32, device=dev)
    n_miss = torch.zeros((4,), dtype=torch.int32, device=dev) if n_miss is None else n_miss
    y = torch.empty_like(x) if y is None else y
    for name, t, dt in (("idx", idx, torch.int32), ("w", w, torch.float32),
                        ("slot", slot, torch.int32)):
        _dev(_shape(t, (T, k), name), dt, name)
    _dev(_at_least(miss_expert, n, "miss_expert"), torch.int32, "miss_expert")
    if miss_pair is not None:
        _dev(_at_least(miss_pair, n, "miss_pair"), torch.int32, "miss_pair")
    _dev(_at_least(n_miss, 2, "n_miss"), torch.int32, "n_miss")
    _dev(_shape(y, tuple(x.shape), "y"), torch.float32, "y")
    L = layer.c_struct()
    if ws is _NO_WS:   # moe_decode_layer_noalloc: the library's own scratch
        _check(lib().moe_decode_layer_noalloc(ctypes.byref(L), _ptr(x), T, _ptr(logits),
                                              _ptr(slot_of_expert), _ptr(idx), _ptr(w),
                                              _ptr(slot), _ptr(miss_expert), _ptr(miss_pair),
                                              _ptr(n_miss), _ptr(y), _stream(stream)),
               "moe_decode_layer_noalloc")
        return y, idx, w, slot, miss_expert, miss_pair, n_miss
    if ws is None:
        ws = torch.empty((decode_workspace_bytes(layer, T),), dtype=torch.uint8, device=dev)
    _check(lib().moe_decode_layer(ctypes.byref(L), _ptr(x), T, _ptr(logits),
                                  _ptr(slot_of_expert), _ptr(idx), _ptr(w), _ptr(slot),
                                  _ptr(miss_expert), _ptr(miss_pair), _ptr(n_miss), _ptr(y),
                                  _ptr(ws), ws.numel(), _stream(stream)), "moe_decode_layer")
    return y, idx, w, slot, miss_expert, miss_pair, n_miss


_NO_WS = object()


def decode_layer_noalloc(layer: MoeLayer, x, logits, slot_of_expert, idx=None, w=None, slot=None,
                         miss_expert=None, miss_pair=None, n_miss=None, y=None, want_pairs=True,
                         stream=None):
    """decode_layer through moe_decode_layer_noalloc (no workspace: the
    library's own scratch array).  Outputs not given are allocated here, by
    torch; pass every output to allocate nothing."""
    return decode_layer(layer, x, logits, slot_of_expert, idx=idx, w=w, slot=slot,
                        miss_expert=miss_expert, miss_pair=miss_pair, n_miss=n_miss, y=y,
                        ws=_NO_WS, want_pairs=want_pairs, stream=stream)


def decode_stack_workspace_bytes(d_model, d_ff, n_experts, top_k, T) -> int:
    return int(lib().moe_decode_stack_workspace_bytes(d_model, d_ff, n_experts, top_k, T))


def new_stack_workspace(layers, T: int, device=None):
    """A workspace for decode_stack over layers of the shape of layers[0]."""
    L0 = layers[0]
    nb = decode_stack_workspace_bytes(L0.d_model, L0.d_ff, L0.n_experts, L0.top_k, T)
    if nb == 0:
        raise ValueError("decode_stack: sizes out of range")
    return torch.empty((nb,), dtype=torch.uint8, device=L0.pool.device if device is None else device)


def decode_stack(layers, x, logits, tables, addends=None, ys=None, routing=False, ws=None,
                 stream=None):
    """Decode / verify through a stack of layers in one call (moe_decode_stack).

    layers: list of MoeLayer (same d_model, d_ff, n_experts, top_k; formats may
    differ); x fp32 [T, d_model]; logits fp32 [L, T, E] (or a list of [T, E]);
    tables: list of int32 [E] slot tables; addends: None or fp32 [L, T, d]
    (entry 0 unused).  ys: fp32 [L, T, d] outputs (allocated if None), or
    fp32 [T, d] for the last layer's output only.  With routing=True also
    returns idx, w, slot [L, T, k], miss_expert, miss_pair [L, T*k] and
    n_miss [L, 4].  Returns a dict."""
    nl = len(layers)
    if nl < 1:
        raise ValueError("decode_stack: at least one layer")
    L0 = layers[0]
    d, f, E, k = L0.d_model, L0.d_ff, L0.n_experts, L0.top_k
    for Lx in layers:
        if (Lx.d_model, Lx.d_ff, Lx.n_experts, Lx.top_k) != (d, f, E, k):
            raise ValueError("decode_stack: every layer needs the same d_model, d_ff, n_experts, top_k")
    _dev(_shape(x, (None, d), "x"), torch.float32, "x")
    T = x.shape[0]
    dev = x.device
    if len(logits) != nl or len(tables) != nl:
        raise ValueError("decode_stack: one logits tensor and one table per layer")
    for l in range(nl):
        _dev(_shape(logits[l], (T, E), f"logits[{l}]"), torch.float32, f"logits[{l}]")
        _dev(_shape(tables[l], (E,), f"tables[{l}]"), torch.int32, f"tables[{l}]")
    if addends is not None:
        if len(addends) != nl:
            raise ValueError("decode_stack: one addend per layer")
        for l in range(nl):
            _dev(_shape(addends[l], (T, d), f"addends[{l}]"), torch.float32, f"addends[{l}]")
    if ys is None:
        ys = torch.empty((nl, T, d), dtype=torch.float32, device=dev)
    last_only = ys.dim() == 2
    _dev(_shape(ys, (T, d) if last_only else (nl, T, d), "ys"), torch.float32, "ys")
    out = {"y": ys}
    if routing:
        # per-layer rows padded to 16 bytes (every pointer must be 16-byte aligned)
        n = T * k
        pad = (n + 3) // 4 * 4

        def rows(dtype, fill):
            buf = torch.full((nl, pad), fill, dtype=dtype, device=dev)
            return buf[:, :n]

        out["idx"] = rows(torch.int32, 0).unflatten(1, (T, k))
        out["w"] = rows(torch.float32, 0).unflatten(1, (T, k))
        out["slot"] = rows(torch.int32, 0).unflatten(1, (T, k))
        out["miss_expert"] = rows(torch.int32, -1)
        out["miss_pair"] = rows(torch.int32, -1)
        out["n_miss"] = torch.zeros((nl, 4), dtype=torch.int32, device=dev)
    if ws is None:
        ws = new_stack_workspace(layers, T)
    _dev(ws, torch.uint8, "ws")
    arr = (MoeStackLayerC * nl)()
    for l, Lx in enumerate(layers):
        _dev(Lx.pool, torch.uint8, "pool")
        n_slots, sb = Lx.pool.shape
        c = arr[l]
        c.pool, c.slot_bytes, c.n_slots, c.fmt = Lx.pool.data_ptr(), sb, n_slots, Lx.fmt
        c.shared_slot, c.reserved = Lx.shared_slot, 0
        c.slot_of_expert, c.logits = tables[l].data_ptr(), logits[l].data_ptr()
        c.addend = addends[l].data_ptr() if (addends is not None and l > 0) else None
        if last_only:
            c.y = ys.data_ptr() if l + 1 == nl else None
        else:
            c.y = ys[l].data_ptr()
        if routing:
            c.idx, c.w, c.slot = (out["idx"][l].data_ptr(), out["w"][l].data_ptr(),
                                  out["slot"][l].data_ptr())
            c.miss_expert, c.miss_pair = out["miss_expert"][l].data_ptr(), out["miss_pair"][l].data_ptr()
            c.n_miss = out["n_miss"][l].data_ptr()
    _check(lib().moe_decode_stack(d, f, E, k, T, nl, arr, _ptr(x), _ptr(ws), ws.numel(),
                                  _stream(stream)), "moe_decode_stack")
    out["ws"] = ws
    return out


@dataclasses.dataclass
class HostTier:
    """A layer's experts in pinned host memory that the GPU reads directly
    (the tier the GPU cache's misses are computed from)."""
    d_model: int
    d_ff: int
    n_experts: int
    top_k: int
    fmt: int
    pool: torch.Tensor            # uint8 [n_slots, slot_bytes], pinned host (or device) memory

    def __post_init__(self):
        if self.pool.dtype != torch.uint8 or self.pool.dim() != 2 or not self.pool.is_contiguous():
            raise ValueError("host tier pool: contiguous uint8 [n_slots, slot_bytes] expected")
        if not (self.pool.is_cuda or self.pool.is_pinned()):
            raise ValueError("host tier pool: pinned host memory or device memory expected")

    def c_struct(self) -> MoeLayerC:
        n_slots, sb = self.pool.shape
        return MoeLayerC(self.d_model, self.d_ff, self.n_experts, self.top_k, self.fmt,
                         n_slots, -1, 0, sb, self.pool.data_ptr())


MISSES_READ, MISSES_JOIN = 1, 2   # phases of moe_decode_misses_phases


def decode_misses(tier: HostTier, x, idx, slot, w, host_slot_of_expert, y, max_rank=None,
                  ws=None, stream=None, phases=MISSES_READ | MISSES_JOIN):
    """Add the missed pairs of a decode step, computed from the host tier,
    into y (moe_decode_misses).  y holds the GPU part on entry.  Returns y.
    phases: MISSES_READ (the products into ws; y, w unused and may be None),
    MISSES_JOIN (y += the products in ws; x may be None), or both
    (moe_decode_misses_phases)."""
    T = (x if x is not None else y).shape[0]
    k = tier.top_k
    read, join = bool(phases & MISSES_READ), bool(phases & MISSES_JOIN)
    checks = [(idx, (T, k), torch.int32, "idx"), (slot, (T, k), torch.int32, "slot"),
              (host_slot_of_expert, (tier.n_experts,), torch.int32, "host_slot_of_expert")]
    if read or x is not None:
        checks.append((x, (T, tier.d_model), torch.float32, "x"))
    if join:
        checks += [(w, (T, k), torch.float32, "w"), (y, (T, tier.d_model), torch.float32, "y")]
    for t, shp, dt, name in checks:   # every shape first, then the devices and types
        _shape(t, shp, name)
    for t, shp, dt, name in checks:
        _dev(t, dt, name)
    r = k if max_rank is None else int(max_rank)
    L = tier.c_struct()
    if ws is None:
        ws = torch.empty((int(lib().moe_decode_workspace_bytes(ctypes.byref(L), T)),),
                         dtype=torch.uint8, device=idx.device)
    _check(lib().moe_decode_misses_phases(ctypes.byref(L), _ptr(x), T, _ptr(idx), _ptr(slot),
                                          _ptr(w), _ptr(host_slot_of_expert), r, _ptr(y),
                                          _ptr(ws), ws.numel(), int(phases), _stream(stream)),
           "moe_decode_misses_phases")
    return y


def decode_layer_tiers(layer: MoeLayer, tier: HostTier, x, logits, slot_of_expert,
                       host_slot_of_expert, max_rank=None, idx=None, w=None, slot=None,
                       miss_expert=None, miss_pair=None, n_miss=None, y=None, ws=None,
                       want_pairs=True, stream=None):
    """Route, look up and run one decode layer with the misses read from the
    host tier in the same launch (moe_decode_layer_tiers).
    Returns (y, idx, w, slot, miss_expert, miss_pair, n_miss)."""
    _shape(x, (None, layer.d_model), "x")
    T = x.shape[0]
    k = layer.top_k
    checks = [(x, torch.float32, "x"),
              (_shape(logits, (T, layer.n_experts), "logits"), torch.float32, "logits"),
              (_shape(slot_of_expert, (layer.n_experts,), "slot_of_expert"), torch.int32,
               "slot_of_expert"),
              (_shape(host_slot_of_expert, (tier.n_experts,), "host_slot_of_expert"),
               torch.int32, "host_slot_of_expert")]
    for t, dt, name in checks:   # every shape above first, then the devices and types
        _dev(t, dt, name)
    dev = x.device
    n = T * k
    idx = torch.empty((T, k), dtype=torch.int32, device=dev) if idx is None else idx
    w = torch.empty((T, k), dtype=torch.float32, device=dev) if w is None else w
    slot = torch.empty((T, k), dtype=torch.int32, device=dev) if slot is None else slot
    if miss_expert is None:
        miss_expert = torch.full((n,), -1, dtype=torch.int32, device=dev)
    if want_pairs and miss_pair is None:
        miss_pair = torch.full((n,), -1, dtype=torch.int32, device=dev)
    n_miss = torch.zeros((4,), dtype=torch.int32, device=dev) if n_miss is None else n_miss
    y = torch.empty_like(x) if y is None else y
    for name, t, dt in (("idx", idx, torch.int32), ("w", w, torch.float32),
                        ("slot", slot, torch.int32)):
        _dev(_shape(t, (T, k), name), dt, name)
    _dev(_at_least(miss_expert, n, "miss_expert"), torch.int32, "miss_expert")
    if miss_pair is not None:
        _dev(_at_least(miss_pair, n, "miss_pair"), torch.int32, "miss_pair")
    _dev(_at_least(n_miss, 2, "n_miss"), torch.int32, "n_miss")
    _dev(_shape(y, tuple(x.shape), "y"), torch.float32, "y")
    if ws is None:
        ws = torch.empty((decode_workspace_bytes(layer, T),), dtype=torch.uint8, device=dev)
    r = k if max_rank is None else int(max_rank)
    L, H = layer.c_struct(), tier.c_struct()
    _check(lib().moe_decode_layer_tiers(ctypes.byref(L), ctypes.byref(H),
                                        _ptr(host_slot_of_expert), r, _ptr(x), T, _ptr(logits),
                                        _ptr(slot_of_expert), _ptr(idx), _ptr(w), _ptr(slot),
                                        _ptr(miss_expert), _ptr(miss_pair), _ptr(n_miss),
                                        _ptr(y), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_decode_layer_tiers")
    return y, idx, w, slot, miss_expert, miss_pair, n_miss


def cache_count(idx, counts, stream=None):
    """counts[e] += uses of expert e in idx (moe_cache_count).  counts: int32
    tensor viewed as uint32 [E]."""
    _dev(idx, torch.int32, "idx")
    _dev(_shape(counts, (None,), "counts"), torch.int32, "counts")
    _check(lib().moe_cache_count(_ptr(idx), idx.numel(), counts.numel(), _ptr(counts),
                                 _stream(stream)), "moe_cache_count")
    return counts


def cache_plan(counts, slot_of_expert, expert_of_slot, shared_slot, host_slot_of_expert,
               host_n_slots, max_swaps, decay_shift=1, swaps=None, n_swaps=None, stream=None):
    """Plan up to max_swaps swaps, updating the tables and decaying the
    counts in place (moe_cache_plan).  Returns (swaps [max_swaps, 4], n_swaps [4])."""
    E = counts.numel()
    for t, name in ((counts, "counts"), (slot_of_expert, "slot_of_expert"),
                    (host_slot_of_expert, "host_slot_of_expert")):
        _shape(t, (E,), name)
    _shape(expert_of_slot, (None,), "expert_of_slot")
    for t, name in ((counts, "counts"), (slot_of_expert, "slot_of_expert"),
                    (expert_of_slot, "expert_of_slot"), (host_slot_of_expert, "host_slot_of_expert")):
        _dev(t, torch.int32, name)
    dev = counts.device
    swaps = torch.full((max_swaps, 4), -1, dtype=torch.int32, device=dev) if swaps is None else swaps
    n_swaps = torch.zeros((4,), dtype=torch.int32, device=dev) if n_swaps is None else n_swaps
    _dev(_shape(swaps, (max_swaps, 4), "swaps"), torch.int32, "swaps")
    _dev(_at_least(n_swaps, 1, "n_swaps"), torch.int32, "n_swaps")
    _check(lib().moe_cache_plan(_ptr(counts), counts.numel(), _ptr(slot_of_expert),
                                _ptr(expert_of_slot), expert_of_slot.numel(), shared_slot,
                                _ptr(host_slot_of_expert), host_n_slots, max_swaps, decay_shift,
                                _ptr(swaps), _ptr(n_swaps), _stream(stream)), "moe_cache_plan")
    return swaps, n_swaps


def cache_fill(layer: MoeLayer, tier: HostTier, swaps, n_swaps, stream=None):
    """Copy the planned experts from the host tier into the cache's slots
    (moe_cache_fill)."""
    _dev(_shape(swaps, (None, 4), "swaps"), torch.int32, "swaps")
    _dev(_at_least(n_swaps, 1, "n_swaps"), torch.int32, "n_swaps")
    L, H = layer.c_struct(), tier.c_struct()
    _check(lib().moe_cache_fill(ctypes.byref(L), ctypes.byref(H), _ptr(swaps), _ptr(n_swaps),
                                swaps.shape[0], _stream(stream)), "moe_cache_fill")


def cache_commit(slot_of_expert, swaps, n_swaps, stream=None):
    """Make the admitted experts visible in the slot table (moe_cache_commit)."""
    _dev(_shape(slot_of_expert, (None,), "slot_of_expert"), torch.int32, "slot_of_expert")
    _dev(_shape(swaps, (None, 4), "swaps"), torch.int32, "swaps")
    _dev(_at_least(n_swaps, 1, "n_swaps"), torch.int32, "n_swaps")
    _check(lib().moe_cache_commit(_ptr(slot_of_expert), slot_of_expert.numel(), _ptr(swaps),
                                  _ptr(n_swaps), swaps.shape[0], _stream(stream)),
           "moe_cache_commit")


def stage_layer(cache: MoeLayer, slot_of_expert, tier: HostTier, host_slot_of_expert, staging,
                stream=None):
    """Copy every expert of the layer into `staging` in expert order
    (moe_stage_layer).  slot_of_expert / host_slot_of_expert: host int32
    arrays [n_experts]; staging: device uint8 [(n_experts + 1), slot_bytes].
    Returns the MoeLayer that reads the staged pool."""
    import numpy as np
    soe = np.ascontiguousarray(np.asarray(slot_of_expert, dtype=np.int32))
    hs = np.ascontiguousarray(np.asarray(host_slot_of_expert, dtype=np.int32))
    for a, name in ((soe, "slot_of_expert"), (hs, "host_slot_of_expert")):
        if a.shape != (cache.n_experts,):
            raise ValueError(f"{name}: shape ({cache.n_experts},) expected, got {a.shape}")
    _dev(staging, torch.uint8, "staging")
    C, H = cache.c_struct(), tier.c_struct()
    _check(lib().moe_stage_layer(ctypes.byref(C), soe.ctypes.data, ctypes.byref(H), hs.ctypes.data,
                                 _ptr(staging), staging.numel(), _stream(stream)),
           "moe_stage_layer")
    return MoeLayer(cache.d_model, cache.d_ff, cache.n_experts, cache.top_k, cache.fmt, staging,
                    cache.n_experts if cache.shared_slot >= 0 else -1)


def prefill_workspace_bytes(layer: MoeLayer, T: int) -> int:
    L = layer.c_struct()
    return int(lib().moe_prefill_workspace_bytes(ctypes.byref(L), T))


def expert_ffn_prefill(layer: MoeLayer, x_bf16, idx, slot, out_pairs=None, pair_pos=None,
                       expert_offsets=None, out_shared=None, with_shared=True, ws=None,
                       stream=None):
    _dev(_shape(x_bf16, (None, layer.d_model), "x_bf16"), torch.bfloat16, "x_bf16")
    T, d = x_bf16.shape
    k = layer.top_k
    _dev(_shape(idx, (T, k), "idx"), torch.int32, "idx")
    _dev(_shape(slot, (T, k), "slot"), torch.int32, "slot")
    dev = x_bf16.device
    if out_pairs is None:
        out_pairs = torch.empty((T * k, d), dtype=torch.float32, device=dev)
    if pair_pos is None:
        pair_pos = torch.empty((T, k), dtype=torch.int32, device=dev)
    if expert_offsets is None:
        expert_offsets = torch.empty((layer.n_experts + 1,), dtype=torch.int32, device=dev)
    if with_shared and layer.shared_slot >= 0 and out_shared is None:
        out_shared = torch.empty((T, d), dtype=torch.float32, device=dev)
    if not with_shared:
        out_shared = None
    if ws is None:
        ws = torch.empty((prefill_workspace_bytes(layer, T),), dtype=torch.uint8, device=dev)
    _dev(_shape(out_pairs, (T * k, d), "out_pairs"), torch.float32, "out_pairs")
    _dev(_shape(pair_pos, (T, k), "pair_pos"), torch.int32, "pair_pos")
    _dev(_shape(expert_offsets, (layer.n_experts + 1,), "expert_offsets"), torch.int32,
         "expert_offsets")
    if out_shared is not None:
        _dev(_shape(out_shared, (T, d), "out_shared"), torch.float32, "out_shared")
    _dev(ws, torch.uint8, "ws")
    L = layer.c_struct()
    _check(lib().moe_expert_ffn_prefill(ctypes.byref(L), _ptr(x_bf16), T, _ptr(idx), _ptr(slot),
                                        _ptr(out_pairs), _ptr(pair_pos), _ptr(expert_offsets),
                                        _ptr(out_shared), _ptr(ws), ws.numel(),
                                        _stream(stream)), "moe_expert_ffn_prefill")
    return out_pairs, pair_pos, expert_offsets, out_shared


def combine(x, rows, pair_pos, w, shared=None, y=None, stream=None):
    if x.dtype == torch.float32:
        x_dtype = DTYPE_F32
    elif x.dtype == torch.bfloat16:
        x_dtype = DTYPE_BF16
    else:
        raise ValueError("x must be float32 or bfloat16")
    _dev(_shape(x, (None, None), "x"), x.dtype, "x")
    T, d = x.shape
    k = pair_pos.shape[1] if pair_pos is not None else 0
    if k:
        _dev(_shape(pair_pos, (T, k), "pair_pos"), torch.int32, "pair_pos")
        _dev(_shape(w, (T, k), "w"), torch.float32, "w")
        _dev(_shape(rows, (None, d), "rows"), torch.float32, "rows")
    if shared is not None:
        _dev(_shape(shared, (T, d), "shared"), torch.float32, "shared")
    if y is None:
        y = torch.empty((T, d), dtype=torch.float32, device=x.device)
    _dev(_shape(y, (T, d), "y"), torch.float32, "y")
    _check(lib().moe_combine(_ptr(x), x_dtype, T, d, k, _ptr(rows), _ptr(pair_pos), _ptr(w),
                             _ptr(shared), _ptr(y), _stream(stream)), "moe_combine")
    return y
