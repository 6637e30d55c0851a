"""Pins of the oracle's unpacker (CPU).

* hand-built slots with closed-form values (tests/golden/*.txt)
* the generator's quantizer + packer round-trips through the oracle's own
  unpacker within the format's rounding bound
"""
import glob
import os

import numpy as np
import pytest
import torch

import oracle
import synth

FMTS = {"Q2S": oracle.FMT_Q2S, "Q2SM": oracle.FMT_Q2SM, "Q3G": oracle.FMT_Q3G}


def _parse(path):
    spec = {"writes": [], "expect": []}
    for raw in open(path):
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        tok = line.split()
        if tok[0] == "format":
            spec["fmt"] = FMTS[tok[1]]
        elif tok[0] == "size":
            spec["size"] = int(tok[1])
        elif tok[0] == "write":
            spec["writes"].append((int(tok[1]), bytes.fromhex(tok[2])))
        elif tok[0] == "expect_block_rl":
            vals = []
            rest = tok[4:]
            for j in range(0, len(rest), 2):
                vals += [float(rest[j])] * int(rest[j + 1].lstrip("x"))
            assert len(vals) == 32, path
            spec["expect"].append((tok[1], int(tok[2]), int(tok[3]), np.array(vals)))
        elif tok[0] == "expect_block":
            pat = [float(v) for v in tok[4:]]
            assert 32 % len(pat) == 0
            spec["expect"].append((tok[1], int(tok[2]), int(tok[3]),
                                   np.array(pat * (32 // len(pat)))))
        else:
            raise ValueError(line)
    return spec


GOLDEN = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "*.txt")))


@pytest.mark.parametrize("path", GOLDEN, ids=[os.path.basename(p) for p in GOLDEN])
def test_hand_built_blocks(path):
    spec = _parse(path)
    d = f = 64
    assert oracle.slot_size(spec["fmt"], d, f) == spec["size"]
    slot = np.zeros(spec["size"], dtype=np.uint8)
    for off, data in spec["writes"]:
        slot[off:off + len(data)] = np.frombuffer(data, dtype=np.uint8)
    mats = {m: oracle.unpack_matrix(slot, spec["fmt"], d, f, m) for m in "GD"}
    named = set()
    for m, row, blk, vals in spec["expect"]:
        np.testing.assert_array_equal(mats[m][row, 32 * blk:32 * blk + 32], vals)
        named.add((m, row, blk))
    for m in "GD":
        for r in range(mats[m].shape[0]):
            for b in range(2):
                if (m, r, b) not in named:
                    assert not mats[m][r, 32 * b:32 * b + 32].any(), (m, r, b)


def test_plane_offsets_against_generator_layout():
    # two independent layout implementations must agree
    for fmt in FMTS.values():
        for d, f in ((64, 64), (256, 128), (2048, 768), (64, 96)):
            lay = synth.slot_layout(fmt, d, f)
            offs = oracle.plane_offsets(fmt, d, f)
            assert lay["total"] == offs["end"]
            for key, val in lay.items():
                if key != "total":
                    assert offs[key] == val[0], (fmt, d, f, key)


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_quantizer_roundtrip(fmt):
    """synth quantize+pack -> oracle unpack stays within half a step."""
    d, f = 256, 96
    gen = torch.Generator().manual_seed(1234 + fmt)
    G = torch.randn(2, 2 * f, d, generator=gen) * 0.02
    D = torch.randn(2, d, f, generator=gen) * 0.02
    G[0, 5, :32] = 0.0                     # an all-zero block: scale 0
    slots = synth.pack_expert_slots(G, D, fmt).numpy()
    for n in range(2):
        for which, W in (("G", G[n]), ("D", D[n])):
            deq = oracle.unpack_matrix(slots[n], fmt, d, f, which)
            w = W.double().numpy()
            blk = w.reshape(w.shape[0], -1, 32)
            if fmt == 1:
                step = np.abs(blk).max(-1) / 1.5
                bound = step / 2
            elif fmt == 2:
                step = (blk.max(-1) - blk.min(-1)) / 3
                bound = step / 2
            else:
                step = np.abs(blk).max(-1) / 3.5
                bound = step / 2
            err = np.abs(deq.reshape(blk.shape) - blk).max(-1)
            # fp16 rounding of scale/min adds at most ~2^-10 relative per weight
            slack = 3 * 2.0 ** -11 * np.abs(blk).max(-1) + 1e-12
            assert np.all(err <= bound + slack), (fmt, which, (err - bound).max())
    assert not oracle.unpack_matrix(slots[0], fmt, d, f, "G")[5, :32].any()


def test_generator_is_deterministic():
    a = synth.make_layer_pool(0, 0, [0, 3, 63])
    b = synth.make_layer_pool(0, 0, [3])
    assert torch.equal(a[1], b[0])
    assert not torch.equal(a[0], a[1])
