"""GPU parity: the router projection (moe_router_logits) against the oracle.

logits = x . W^T with bfloat16 weights.  The kernel multiplies and adds in
fp32 (each lane in element order, d/64 fused multiply-adds, then a fixed
butterfly of 6 additions); the oracle sums exactly.  Bar per logit:
|got - ref| <= 2 (d/64 + 8) 2^-24 sum_j |x_j w_j|, twice the first-order
bound of that summation.  Two runs must give the same bits.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import need_gpu

pytestmark = pytest.mark.gpu


def _check(T, d, E, cfg, layer):
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    x = synth.make_x(cfg, layer, T, d).to(dev)
    w = synth.make_router_weights(cfg, layer, E, d).to(dev)
    got = bf.router_logits(x, w)
    again = bf.router_logits(x, w)
    torch.cuda.synchronize()
    got, again = got.cpu().numpy(), again.cpu().numpy()
    assert np.array_equal(got, again)
    wb = w.cpu().view(torch.int16).numpy().view(np.uint16)
    xn = x.cpu().numpy()
    ref = oracle.router_logits(xn, wb)
    mag = np.abs(xn.astype(np.float64)) @ np.abs(oracle.bf16_bits_to_f64(wb)).T
    bound = 2.0 * (d / 64 + 8) * 2.0 ** -24 * mag
    err = np.abs(got.astype(np.float64) - ref)
    assert (err <= bound).all(), float((err / np.maximum(bound, 1e-300)).max())
    return got


CASES = [
    # T, d_model, n_experts: the model's router (T = 1 and the verify step),
    # the smallest sizes, and rows that end inside a 512-element pass
    (1, 2048, 512), (4, 2048, 512), (2, 64, 1), (3, 192, 7), (1, 704, 1000), (4, 1024, 1024),
]


@pytest.mark.parametrize("T,d,E", CASES, ids=[f"T{c[0]}_d{c[1]}_E{c[2]}" for c in CASES])
def test_router_logits(T, d, E):
    _check(T, d, E, 5, 7 * T + E)


def test_router_logits_tokens_independent():
    """A token's logits do not depend on the other tokens of the step: the
    T = 4 call gives, bit for bit, the logits of four T = 1 calls."""
    import bit_expert_ffn_top_amd as bf
    dev = need_gpu()
    d, E = 2048, 512
    x = synth.make_x(6, 1, 4, d).to(dev)
    w = synth.make_router_weights(6, 1, E, d).to(dev)
    four = bf.router_logits(x, w)
    ones = torch.cat([bf.router_logits(x[t:t + 1].contiguous(), w) for t in range(4)])
    torch.cuda.synchronize()
    assert torch.equal(four.cpu(), ones.cpu())
