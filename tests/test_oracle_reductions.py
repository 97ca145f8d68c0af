"""Pins for the oracle's fixed-order sums: values whose result depends on the order (so a wrong
tree shape or a missing fused multiply-add fails), and error bounds against exact sums."""
from fractions import Fraction

import numpy as np


def test_tree_order_pin(orc):
    # pairwise: (1e8 + 1) + (-1e8 + 1) = 1e8 + (-1e8) = 0 in binary32; left to right gives 1
    x = np.array([1e8, 1.0, -1e8, 1.0], np.float32)
    assert orc.tree_sum(x) == np.float32(0.0)
    # eight terms: ((a+b)+(c+d)) + ((e+f)+(g+h))
    x = np.array([1.0, 2 ** 24, -(2 ** 24), 1.0, 3.0, 0.0, 0.0, 0.0], np.float32)
    a = np.float32(np.float32(1.0) + np.float32(2 ** 24))
    b = np.float32(np.float32(-(2 ** 24)) + np.float32(1.0))
    assert orc.tree_sum(x) == np.float32(np.float32(a + b) + np.float32(3.0))


def _fma32(a, b, c):
    return np.float32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def _chain(x, y):
    s = np.float32(x[0] * y[0])
    for t in range(1, len(x)):
        s = _fma32(x[t], y[t], s)
    return s


def test_dot_order_pin(orc):
    # blocks of 32: s = x0*y0, then s = fma(x_i, y_i, s) first to last; block sums by tree()
    g = np.random.default_rng(7)
    for n in (8, 32, 64, 128):
        for _ in range(40):
            x = g.standard_normal(n).astype(np.float32)
            y = g.standard_normal(n).astype(np.float32)
            blocks = [_chain(x[i:i + 32], y[i:i + 32]) for i in range(0, n, 32)]
            assert orc.dot(x, y) == orc.tree_sum(np.array(blocks, np.float32))
    # a case where the fused and the separately rounded evaluation differ
    x = np.array([1.0, 1 + 2 ** -12, 0, 0], np.float32)
    y = np.array([-1.0, 1 + 2 ** -12, 0, 0], np.float32)
    fused = np.float32(Fraction(float(x[1])) ** 2 - 1)
    assert orc.dot(x, y) == fused
    assert fused != np.float32(np.float32(x[1] * y[1]) - np.float32(1.0))
    # one chain over 64 terms and two chains of 32 added differ: after 2^24 every +1 of a single
    # chain is a tie that rounds back to 2^24, while the second block sums its 32 ones exactly
    x = np.zeros(64, np.float32)
    x[0] = 2.0 ** 24
    x[32:] = 1.0
    y = np.ones(64, np.float32)
    assert _chain(x, y) == np.float32(2.0 ** 24)
    assert orc.dot(x, y) == np.float32(2.0 ** 24 + 32)


def test_sums_within_error_bound(orc):
    g = np.random.default_rng(3)
    u = 2.0 ** -24
    for n in (4, 8, 64, 128):
        for _ in range(50):
            x = g.standard_normal(n).astype(np.float32)
            y = g.standard_normal(n).astype(np.float32)
            exact = float(sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x, y)))
            depth = min(n, 32) + max(0, int(np.log2(n / 32)))
            bound = depth * u * float(np.sum(np.abs(x.astype(np.float64) * y)))
            assert abs(float(orc.dot(x, y)) - exact) <= bound
            ex = float(sum(Fraction(float(a)) for a in x))
            assert abs(float(orc.tree_sum(x)) - ex) <= np.log2(n) * u * float(np.sum(np.abs(x)))
