"""Seeded generator, block quantizer and slot packer.

Everything here produces inputs.  There are five layer workloads (a tiny
plumbing layer; one decode layer at the model's counts; the expert-cache
hit/miss layer; the 1+3-token verify step; the 8,192-token prefill chunk).  The model counts behind them -- 48 layers,
512 routed experts per layer, 10 chosen per token plus one shared expert --
are given in "Strata" (news.blueqat.app post 3262), section "Strataとは".

Packed slot layout (the byte format both the oracle and the HIP library read;
each implements its own reader):

* An expert slot holds two matrices, G then D.
  - G has 2*d_ff rows and d_model columns; row 2j is the gate row j and row
    2j+1 is the up row j.
  - D has d_model rows and d_ff columns (the down projection).
* Rows are cut into blocks of 32 consecutive weights.  A matrix is stored in
  units of U consecutive blocks of one row (U = 2 for G, U = 1 for D); with R
  rows, unit c of row r has index c*R + r, so one unit of 64 consecutive rows
  is contiguous.  Each matrix is a sequence of planes, each starting on a
  256-byte boundary measured from the slot start, each holding the units in
  index order:
  - codes: 8 bytes per block; code i of the block sits at bits [2i, 2i+2) of
    the little-endian 64-bit word (for the 3-bit format: the low two bits).
  - hi (3-bit format only): 4 bytes per block, a little-endian 32-bit word in
    which bit 2i+1 is bit 2 of code i for i < 16 and bit 2(i-16) is bit 2 of
    code i for i >= 16.
  - scale: one IEEE fp16 per block.
  - min (2-bit scale+min format only): one IEEE fp16 per block.
  Inside a unit the U blocks follow each other in every plane.
* The slot size is rounded up to 256 bytes.

Formats and how a code decodes (the quantizer below only has to produce codes
that decode this way):
  Q2S  (1): w = s * (q - 1.5), q in 0..3                   -> 10 B / 32 w
  Q2SM (2): w = m + s * q,     q in 0..3                   -> 12 B / 32 w
  Q3G  (3): w = s * g[q] / 3.5, g = -3.5..3.5 step 1, q 0..7 -> 14 B / 32 w
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

BASE_SEED = 20261203
FMT_Q2S, FMT_Q2SM, FMT_Q3G = 1, 2, 3
BLOCK = 32
ALIGN = 256

# tags that separate the seeded streams
TAG_W, TAG_X, TAG_LOGITS, TAG_SLOTS, TAG_ZIPF, TAG_RESIDENT = 1, 2, 3, 4, 5, 6
TAG_ROUTER = 7


@dataclasses.dataclass(frozen=True)
class LayerShape:
    n_experts: int
    top_k: int
    d_model: int
    d_ff: int
    shared: bool


# Workload table.  `fmt` may be a tuple that alternates by layer index.
WORKLOADS = {
    0: dict(shape=LayerShape(64, 4, 256, 128, False), T=1, fmt=FMT_Q2S,
            logit_sigma=1.0, n_layers=1, x_dtype="f32", routing="normal",
            resident="all_identity"),
    1: dict(shape=LayerShape(512, 10, 2048, 768, True), T=1, fmt=FMT_Q2SM,
            logit_sigma=1.5, n_layers=48, x_dtype="f32", routing="normal",
            resident="all_permuted"),
    2: dict(shape=LayerShape(512, 10, 2048, 768, True), T=1, fmt=FMT_Q2SM,
            logit_sigma=None, n_layers=48, x_dtype="f32", routing="zipf",
            resident="zipf94", zipf_s=1.1, n_resident=94, n_top_resident=62),
    3: dict(shape=LayerShape(512, 10, 2048, 768, True), T=4,
            fmt=(FMT_Q2SM, FMT_Q3G), logit_sigma=1.5, n_layers=48,
            x_dtype="f32", routing="normal", resident="all_permuted"),
    4: dict(shape=LayerShape(512, 10, 2048, 768, True), T=8192, fmt=FMT_Q2SM,
            logit_sigma=1.5, n_layers=48, x_dtype="bf16", routing="normal",
            resident="all_permuted"),
}


def config_shape(cfg: int) -> LayerShape:
    return WORKLOADS[cfg]["shape"]


def layer_format(cfg: int, layer: int) -> int:
    fmt = WORKLOADS[cfg]["fmt"]
    if isinstance(fmt, tuple):
        return fmt[layer % len(fmt)]
    return fmt


def seed_of(cfg: int, layer: int, expert: int, tag: int, extra: int = 0) -> int:
    """63-bit seed for one stream; expert -1 means 'not per expert'."""
    ss = np.random.SeedSequence([BASE_SEED, cfg, layer, expert + 1, tag, extra])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(2**63 - 1))


def torch_gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


# --------------------------------------------------------------------------
# slot layout (byte offsets of each plane)
# --------------------------------------------------------------------------

def _align(n: int) -> int:
    return (n + ALIGN - 1) // ALIGN * ALIGN


def _planes(fmt: int):
    if fmt == FMT_Q2S:
        return [("codes", 8), ("scale", 2)]
    if fmt == FMT_Q2SM:
        return [("codes", 8), ("scale", 2), ("min", 2)]
    if fmt == FMT_Q3G:
        return [("codes", 8), ("hi", 4), ("scale", 2)]
    raise ValueError(f"unknown format {fmt}")


UNIT_BLOCKS = {"G": 2, "D": 1}


def slot_layout(fmt: int, d_model: int, d_ff: int) -> dict:
    """{('G'|'D', plane): (offset, bytes)} plus 'total'."""
    out = {}
    off = 0
    for mat, rows, cols in (("G", 2 * d_ff, d_model), ("D", d_model, d_ff)):
        nblk = rows * (cols // BLOCK)
        for name, per in _planes(fmt):
            out[(mat, name)] = (off, nblk * per)
            off = _align(off + nblk * per)
    out["total"] = off
    return out


def slot_bytes(fmt: int, d_model: int, d_ff: int) -> int:
    return slot_layout(fmt, d_model, d_ff)["total"]


# --------------------------------------------------------------------------
# quantizer (input generation: maps fp32 weights to codes + fp16 params)
# --------------------------------------------------------------------------

def quantize_blocks(w: torch.Tensor, fmt: int):
    """w: float32 [..., 32].  Returns (codes uint8 [..., 32], scale fp16 [...],
    min fp16 [...] or None)."""
    assert w.dtype == torch.float32 and w.shape[-1] == BLOCK
    zero = torch.zeros((), dtype=torch.float32, device=w.device)
    if fmt == FMT_Q2S:
        s16 = (w.abs().amax(-1) / 1.5).to(torch.float16)
        s = s16.float().unsqueeze(-1)
        q = torch.where(s > 0, torch.round(w / torch.where(s > 0, s, 1.0) + 1.5), zero)
        return q.clamp_(0, 3).to(torch.uint8), s16, None
    if fmt == FMT_Q2SM:
        mn = w.amin(-1)
        mx = w.amax(-1)
        m16 = mn.to(torch.float16)
        s16 = ((mx - mn) / 3.0).to(torch.float16)
        s = s16.float().unsqueeze(-1)
        m = m16.float().unsqueeze(-1)
        q = torch.where(s > 0, torch.round((w - m) / torch.where(s > 0, s, 1.0)), zero)
        return q.clamp_(0, 3).to(torch.uint8), s16, m16
    if fmt == FMT_Q3G:
        s16 = w.abs().amax(-1).to(torch.float16)
        s = s16.float().unsqueeze(-1)
        q = torch.where(s > 0, torch.round(3.5 * w / torch.where(s > 0, s, 1.0) + 3.5), zero)
        return q.clamp_(0, 7).to(torch.uint8), s16, None
    raise ValueError(f"unknown format {fmt}")


def _hi_bit_positions():
    pos = torch.empty(32, dtype=torch.int64)
    for i in range(32):
        pos[i] = 2 * i + 1 if i < 16 else 2 * (i - 16)
    return pos


def pack_matrix_planes(codes: torch.Tensor, s16: torch.Tensor, m16, fmt: int) -> dict:
    """codes uint8 [..., nb, 32] -> {plane: uint8 tensor [..., nb, per]}
    in the order of the leading dimensions (no unit reordering here)."""
    lead = codes.shape[:-1]  # [..., nb]
    c = codes.to(torch.int32)
    sh2 = torch.tensor([0, 2, 4, 6], dtype=torch.int32, device=codes.device)
    lo = (c & 3).reshape(*lead, 8, 4)
    out = {"codes": (lo << sh2).sum(-1).to(torch.uint8)}                # [..., nb, 8]
    if fmt == FMT_Q3G:
        bit = ((c >> 2) & 1).to(torch.int64)                             # [..., nb, 32]
        pos = _hi_bit_positions().to(codes.device)
        word = (bit << pos).sum(-1)                                      # [..., nb]
        sh = torch.tensor([0, 8, 16, 24], dtype=torch.int64, device=codes.device)
        out["hi"] = ((word.unsqueeze(-1) >> sh) & 255).to(torch.uint8)   # [..., nb, 4]
    out["scale"] = s16.contiguous().view(torch.uint8).reshape(*lead, 2)
    if fmt == FMT_Q2SM:
        out["min"] = m16.contiguous().view(torch.uint8).reshape(*lead, 2)
    return out


def pack_expert_slots(G: torch.Tensor, D: torch.Tensor, fmt: int) -> torch.Tensor:
    """G float32 [n, 2*d_ff, d_model], D float32 [n, d_model, d_ff] ->
    uint8 [n, slot_bytes]."""
    n, rows_g, d = G.shape
    f = rows_g // 2
    assert D.shape == (n, d, f)
    lay = slot_layout(fmt, d, f)
    out = torch.zeros((n, lay["total"]), dtype=torch.uint8, device=G.device)
    for mat, W in (("G", G), ("D", D)):
        rows, cols = W.shape[1], W.shape[2]
        nb = cols // BLOCK
        U = UNIT_BLOCKS[mat]
        codes, s16, m16 = quantize_blocks(W.reshape(n, rows, nb, BLOCK), fmt)
        planes = pack_matrix_planes(codes, s16, m16, fmt)            # [n, rows, nb, per]
        for name, data in planes.items():
            per = data.shape[-1]
            # [n, rows, nb/U, U, per] -> [n, nb/U, rows, U, per]: unit c of row r at c*rows + r
            unit = data.reshape(n, rows, nb // U, U, per).permute(0, 2, 1, 3, 4)
            off, nbytes = lay[(mat, name)]
            flat = unit.reshape(n, -1)
            assert flat.shape[1] == nbytes, (mat, name, flat.shape, nbytes)
            out[:, off:off + nbytes] = flat
    return out


# --------------------------------------------------------------------------
# weights, activations, logits, slot tables
# --------------------------------------------------------------------------

def expert_weights(cfg: int, layer: int, expert: int, shape: LayerShape,
                   device="cpu", sigma: float = 0.02):
    """W_gate [f, d], W_up [f, d], W_down [d, f], float32 ~ N(0, sigma).
    expert == shape.n_experts denotes the shared expert."""
    d, f = shape.d_model, shape.d_ff
    g = torch_gen(seed_of(cfg, layer, expert, TAG_W), device)
    w = torch.randn(3 * f * d, generator=g, dtype=torch.float32, device=device)
    w.mul_(sigma)
    return w[:f * d].view(f, d), w[f * d:2 * f * d].view(f, d), w[2 * f * d:].view(d, f)


def _interleave_gate_up(Wg: torch.Tensor, Wu: torch.Tensor) -> torch.Tensor:
    f, d = Wg.shape
    return torch.stack([Wg, Wu], dim=1).reshape(2 * f, d)


def make_layer_pool(cfg: int, layer: int, experts, device="cpu", fmt=None,
                    batch: int = 32, shape: LayerShape | None = None) -> torch.Tensor:
    """Packed slots for the listed expert ids (n_experts = shared expert),
    in list order: uint8 [len(experts), slot_bytes].  `shape` overrides the
    configuration's layer shape (the seeds still come from `cfg`)."""
    shape = config_shape(cfg) if shape is None else shape
    fmt = layer_format(cfg, layer) if fmt is None else fmt
    sb = slot_bytes(fmt, shape.d_model, shape.d_ff)
    out = torch.empty((len(experts), sb), dtype=torch.uint8, device=device)
    for i0 in range(0, len(experts), batch):
        ids = experts[i0:i0 + batch]
        Gs, Ds = [], []
        for e in ids:
            Wg, Wu, Wd = expert_weights(cfg, layer, int(e), shape, device)
            Gs.append(_interleave_gate_up(Wg, Wu))
            Ds.append(Wd)
        out[i0:i0 + len(ids)] = pack_expert_slots(torch.stack(Gs), torch.stack(Ds), fmt)
        del Gs, Ds
    return out


def make_x(cfg: int, layer: int, T: int, d: int, device="cpu", step: int = 0,
           dtype=torch.float32) -> torch.Tensor:
    """Activations ~ N(0, 1), rounded to `dtype` (bf16 for the prefill chunk)."""
    g = torch_gen(seed_of(cfg, layer, -1, TAG_X, step), device)
    x = torch.randn((T, d), generator=g, dtype=torch.float32, device=device)
    return x.to(dtype)


def make_logits(cfg: int, layer: int, T: int, E: int, sigma: float,
                device="cpu", step: int = 0) -> torch.Tensor:
    """Router logits ~ N(0, sigma), fp32 [T, E]."""
    g = torch_gen(seed_of(cfg, layer, -1, TAG_LOGITS, step), device)
    return torch.randn((T, E), generator=g, dtype=torch.float32, device=device) * sigma


def make_router_weights(cfg: int, layer: int, E: int, d: int, sigma: float = 0.02,
                        device="cpu") -> torch.Tensor:
    """Router projection weights ~ N(0, sigma), bfloat16 [E, d]."""
    g = torch_gen(seed_of(cfg, layer, -1, TAG_ROUTER), device)
    w = torch.randn((E, d), generator=g, dtype=torch.float32, device=device) * sigma
    return w.to(torch.bfloat16)


def _zipf_perm(cfg: int, layer: int, E: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed_of(cfg, layer, -1, TAG_ZIPF)))
    return rng.permutation(E)  # perm[r] = expert holding popularity rank r+1


def zipf_popularity(cfg: int, layer: int, E: int) -> np.ndarray:
    """Expert ids by popularity, most used first, as zipf_gumbel_logits draws them."""
    return _zipf_perm(cfg, layer, E).copy()


def zipf_gumbel_logits(cfg: int, layer: int, T: int, E: int, s: float,
                       device="cpu", step: int = 0) -> torch.Tensor:
    """logit_e = -s*ln(rank(e)) + Gumbel(0,1): the top-k of these is a draw of
    k distinct experts without replacement with weights rank^-s."""
    perm = _zipf_perm(cfg, layer, E)
    rank = np.empty(E, dtype=np.float64)
    rank[perm] = np.arange(1, E + 1)
    base = torch.tensor(-s * np.log(rank), dtype=torch.float32, device=device)
    g = torch_gen(seed_of(cfg, layer, -1, TAG_LOGITS, step), device)
    u = torch.rand((T, E), generator=g, dtype=torch.float32, device=device)
    u = u.clamp_(min=1e-12)
    gumbel = -torch.log((-torch.log(u)).clamp_(min=1e-30))
    return base.unsqueeze(0) + gumbel


def zipf_residency(cfg: int, layer: int, E: int, n_top: int, n_resident: int) -> np.ndarray:
    """Resident expert ids: popularity ranks 1..n_top plus seeded random others."""
    perm = _zipf_perm(cfg, layer, E)
    top = perm[:n_top]
    rng = np.random.Generator(np.random.PCG64(seed_of(cfg, layer, -1, TAG_RESIDENT)))
    rest = rng.choice(perm[n_top:], size=n_resident - n_top, replace=False)
    return np.sort(np.concatenate([top, rest]))


def make_slot_table(cfg: int, layer: int):
    """Returns (slot_of_expert int32 [E], shared_slot, slot_expert list) where
    slot_expert[s] is the expert id stored in slot s (E = shared expert)."""
    c = WORKLOADS[cfg]
    shape = c["shape"]
    E = shape.n_experts
    if c["resident"] == "all_identity":
        resident = np.arange(E)
    elif c["resident"] == "all_permuted":
        resident = np.arange(E)
    elif c["resident"] == "zipf94":
        resident = zipf_residency(cfg, layer, E, c["n_top_resident"], c["n_resident"])
    else:
        raise ValueError(c["resident"])
    ids = list(resident) + ([E] if shape.shared else [])
    n_slots = len(ids)
    if c["resident"] == "all_identity":
        order = np.arange(n_slots)
    else:
        rng = np.random.Generator(np.random.PCG64(seed_of(cfg, layer, -1, TAG_SLOTS)))
        order = rng.permutation(n_slots)  # ids[i] goes to slot order[i]
    slot_expert = [0] * n_slots
    for i, s in enumerate(order):
        slot_expert[int(s)] = int(ids[i])
    slot_of_expert = np.full(E, -1, dtype=np.int32)
    shared_slot = -1
    for s, e in enumerate(slot_expert):
        if e == E:
            shared_slot = s
        else:
            slot_of_expert[e] = s
    return slot_of_expert, shared_slot, slot_expert

