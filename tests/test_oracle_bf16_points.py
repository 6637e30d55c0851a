"""Pins of where the oracle's prefill expert rounds to bfloat16 (CPU).

Reading C16 (prefill chunk precision; the pages only say the prefill runs in
8,192-token chunks on the GPU, "Strata" on news.blueqat.app, section
"GPU・CPU・RAM・SSDの分担"): x enters as bfloat16, every dequantized weight of
W_gate, W_up and W_down is rounded to bfloat16 (nearest, ties to even), the
products are summed wide, h = silu(g) * u is rounded to bfloat16 once, and the
output stays wide.

Each case below is a tiny expert whose weights have the block form m + s*q
(fp16 m and s, 2-bit q) and are not bfloat16 values, so that every one of the
four rounding points changes the result by an amount worked out by hand in
the comments.  The expected outputs are literals; the only library call in
the derivation is math.exp inside silu, and the tests assert that the value
being rounded lies strictly inside the rounding interval the literal assumes.

The mutants are the plausible mistakes: a rounding point dropped, or moved
(g and u rounded instead of h, the output rounded).  Each one is written out
here as a variant of the definition and must miss the expected literals, so
the pins would catch it.
"""
import math

import numpy as np
import pytest

import oracle

BF16_SPACING_1_2 = 2.0 ** -7      # bfloat16 keeps 8 significant bits: spacing on [1, 2)
BF16_SPACING_HALF_1 = 2.0 ** -8   # spacing on [0.5, 1)


def _silu(z):
    return z / (1.0 + math.exp(-z))


def _case_a():
    """One-hot x.

    x = (1, 0).  Gate weight 2 + 2^-10 (m = 2, s = 2^-10, q = 1): on [2, 4)
    the bfloat16 spacing is 2^-6, and 2^-10 is 1/16 of it, so it rounds to
    2.  Up weight 0.5 + 2^-9 (m = 0.5, s = 2^-10, q = 2): exactly half the
    2^-8 spacing above 0.5, a tie, so it rounds to the even neighbour 0.5.
    g = 2, u = 0.5, silu(2) * 0.5 = 1 / (1 + e^-2) = 225.484... * 2^-8, just
    below the tie at 225.5, so h = 225 * 2^-8.
    Down column (1 + 3 * 2^-9, -(0.5 + 2^-10)): 3 * 2^-9 is 0.75 of the 2^-7
    spacing, so the first rounds up to 1 + 2^-7; 2^-10 is a quarter of the
    2^-8 spacing, so the second rounds to -0.5.
    y = (225 * 2^-8 * (1 + 2^-7), -225 * 2^-8 * 0.5)
      = (29025 / 32768, -225 / 512), both exact in float64.
    The second column of W_gate and W_up meets x_1 = 0 and must not matter.
    """
    x = np.array([[1.0, 0.0]])
    Wg = np.array([[2.0 + 2.0 ** -10, 7.0]])
    Wu = np.array([[0.5 + 2.0 * 2.0 ** -10, -3.0]])
    Wd = np.array([[1.0 + 3.0 * 2.0 ** -9], [-(0.5 + 2.0 ** -10)]])
    p = _silu(2.0) * 0.5
    assert 224.5 < p / BF16_SPACING_HALF_1 < 225.5          # h = 225 * 2^-8
    assert abs(p / BF16_SPACING_HALF_1 - 225.5) < 0.02      # and close to the tie above
    y = np.array([[29025.0 / 32768.0, -225.0 / 512.0]])
    return x, Wg, Wu, Wd, y


def _case_b():
    """Two-hot x, so that g is a sum that is not a bfloat16 value.

    x = (1, 1).  Gate row (1 + 3 * 2^-9, 2^-10): the first rounds up to
    1 + 2^-7 (0.75 of the spacing), the second is a power of two (exact).
    g = 1 + 2^-7 + 2^-10 = 1.0087890625 (not a bfloat16 value: it lies a
    eighth of the way from 1 + 2^-7 to 1 + 2^-6).
    Up row (0.5 + 2^-10, 0.5 + 2^-10): each rounds to 0.5 (a quarter of the
    spacing), u = 1.
    silu(1.0087890625) = 189.241... * 2^-8, so h = 189 * 2^-8.  Rounding g
    instead (to 1 + 2^-7) would give silu(1 + 2^-7) = 189.0087 * 2^-8, which
    then stays unrounded: not the literal.
    Down column (1, -0.75), both bfloat16 values: y = (189 / 256, -567 / 1024).
    """
    x = np.array([[1.0, 1.0]])
    Wg = np.array([[1.0 + 3.0 * 2.0 ** -9, 2.0 ** -10]])
    Wu = np.array([[0.5 + 2.0 ** -10, 0.5 + 2.0 ** -10]])
    Wd = np.array([[1.0], [-0.75]])
    g = 1.0 + 2.0 ** -7 + 2.0 ** -10
    p = _silu(g) * 1.0
    assert 188.5 < p / BF16_SPACING_HALF_1 < 189.5           # h = 189 * 2^-8
    y = np.array([[189.0 / 256.0, -567.0 / 1024.0]])
    return x, Wg, Wu, Wd, y


CASES = {"one_hot": _case_a, "two_hot": _case_b}


def _variant(x, Wg, Wu, Wd, *, round_wg=True, round_wu=True, round_wd=True, round_h=True,
             round_gu=False, round_out=False):
    """The definition with each rounding point switchable (mutants only)."""
    r = oracle.bf16_round
    g = x @ (r(Wg) if round_wg else Wg).T
    u = x @ (r(Wu) if round_wu else Wu).T
    if round_gu:
        g, u = r(g), r(u)
    h = oracle.silu(g) * u
    if round_h:
        h = r(h)
    y = h @ (r(Wd) if round_wd else Wd).T
    return r(y) if round_out else y


MUTANTS = {
    "W_down left unrounded": dict(round_wd=False),
    "W_gate left unrounded": dict(round_wg=False),
    "W_up left unrounded": dict(round_wu=False),
    "h left unrounded": dict(round_h=False),
    "g and u rounded instead of h": dict(round_gu=True, round_h=False),
    "output rounded to bfloat16": dict(round_out=True),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_oracle_rounding_points_closed_form(case):
    x, Wg, Wu, Wd, y = CASES[case]()
    got = oracle.expert_ffn_bf16(x, Wg, Wu, Wd)
    np.testing.assert_array_equal(got, y)


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_each_misplaced_rounding_misses_a_literal(mutant):
    missed = []
    for case in sorted(CASES):
        x, Wg, Wu, Wd, y = CASES[case]()
        # the switchable definition with every point in place is the literal
        np.testing.assert_array_equal(_variant(x, Wg, Wu, Wd), y)
        if not np.array_equal(_variant(x, Wg, Wu, Wd, **MUTANTS[mutant]), y):
            missed.append(case)
    assert missed, f"mutant '{mutant}' matches every literal: the pins would not catch it"


def test_prefill_layer_uses_the_same_rounding_points():
    """prefill_layer routes both tokens of case A / case B through one
    expert with weight 1 (k = 1): its pair rows are the literals."""
    xa, Wg, Wu, Wd, ya = _case_a()
    xb, Wg2, Wu2, Wd2, yb = _case_b()
    experts = [(Wg, Wu, Wd), (Wg2, Wu2, Wd2)]
    x = np.concatenate([xa, xb])
    idx = np.array([[0], [1]])
    w = np.array([[1.0], [1.0]])
    out_pairs, out_shared, y = oracle.prefill_layer(x, idx, w, lambda e: experts[e], None, 2)
    assert out_shared is None
    np.testing.assert_array_equal(out_pairs, np.concatenate([ya, yb]))
    np.testing.assert_array_equal(y, x + np.concatenate([ya, yb]))
