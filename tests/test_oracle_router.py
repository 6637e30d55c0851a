"""Pins of the oracle's router projection (router_logits) and of its
bfloat16 decoding, against values fixed by the bfloat16 format and by hand
arithmetic: no test re-computes the oracle's own formula."""
import numpy as np

import oracle


def test_bf16_bit_patterns():
    # sign | 8-bit exponent (bias 127) | 7-bit mantissa
    pats = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x4000, 0xC040, 0x3F00, 0x3FC0,
                     0x4120, 0x7F80, 0xFF80, 0x0001, 0x7F7F], dtype=np.uint16)
    want = [0.0, -0.0, 1.0, -1.0, 2.0, -3.0, 0.5, 1.5, 10.0, np.inf, -np.inf,
            2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127]
    got = oracle.bf16_bits_to_f64(pats)
    for g, w in zip(got, want):
        assert g == w, (g, w)
    assert np.signbit(got[1])
    assert np.isnan(oracle.bf16_bits_to_f64(np.array([0x7FC0], np.uint16))[0])


def test_router_logits_by_hand():
    # W rows (bf16): [1, 0, -1], [0.5, 2, 0], [-3, 1.5, 10]
    w = np.array([[0x3F80, 0x0000, 0xBF80],
                  [0x3F00, 0x4000, 0x0000],
                  [0xC040, 0x3FC0, 0x4120]], dtype=np.uint16)
    x = np.array([[1.0, 2.0, 3.0],
                  [-2.0, 0.25, 4.0]])
    want = np.array([[1 - 3, 0.5 + 4, -3 + 3 + 30],
                     [-2 - 4, -1 + 0.5, 6 + 0.375 + 40]])
    np.testing.assert_array_equal(oracle.router_logits(x, w), want)


def test_router_logits_unit_rows_select_features():
    # row e = unit vector at column c_e (bf16 1.0): logit e is x[:, c_e] exactly
    rng = np.random.default_rng(7)
    T, d, E = 3, 64, 10
    cols = rng.permutation(d)[:E]
    w = np.zeros((E, d), np.uint16)
    w[np.arange(E), cols] = 0x3F80
    x = rng.standard_normal((T, d))
    np.testing.assert_array_equal(oracle.router_logits(x, w), x[:, cols])


def test_router_logits_linear_in_x():
    # integer-valued inputs and power-of-two weights: every sum is exact, so
    # linearity holds to the last bit
    rng = np.random.default_rng(8)
    T, d, E = 2, 128, 16
    exps = rng.integers(120, 134, size=(E, d)).astype(np.uint16)   # 2^-7 .. 2^6
    w = (exps << 7) | (rng.integers(0, 2, size=(E, d)).astype(np.uint16) << 15)
    a = rng.integers(-50, 50, size=(T, d)).astype(np.float64)
    b = rng.integers(-50, 50, size=(T, d)).astype(np.float64)
    la, lb, lab = (oracle.router_logits(v, w) for v in (a, b, a + b))
    np.testing.assert_array_equal(lab, la + lb)
    np.testing.assert_array_equal(oracle.router_logits(3 * a, w), 3 * la)
