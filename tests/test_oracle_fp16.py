"""Pins for the oracle's binary16 conversion against NumPy's IEEE conversion (an independent
library routine): round to nearest even, subnormals, overflow to infinity."""
import numpy as np


def _check(orc, x):
    x = np.asarray(x, np.float32)
    got = orc.f32_to_f16_bits(x)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan]), x[~nan][got[~nan] != ref[~nan]][:10]
    # NaN stays NaN
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)


def test_f16_to_f32_exhaustive(orc):
    h = np.arange(65536, dtype=np.uint16)
    got = orc.f16_bits_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.all(np.isnan(got[nan]))


def test_f32_to_f16_stratified(orc):
    # every combination of the top 16 bits (sign, exponent, 7 mantissa bits) with low halves
    # that sit on, just below and just above the rounding points of binary16
    hi = np.arange(65536, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0x2001, 0x7FFF,
                     0x8000, 0xF000, 0xFFFF], np.uint32)
    x = (hi[:, None] | lows[None, :]).ravel().view(np.float32)
    _check(orc, x)


def test_f32_to_f16_ties_and_boundaries(orc):
    # the exact midpoints between consecutive binary16 values, and one binary32 ulp either side
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)  # exact in binary32
    for x in (mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(np.inf))):
        _check(orc, x)
        _check(orc, -x)
    # overflow threshold: 65520 rounds to infinity, the value just below to 65504
    _check(orc, np.array([65504, 65519.996, 65520, 1e30, np.inf, -np.inf, 2 ** -25,
                          np.float32(2 ** -25) * np.float32(1.0000001), 2 ** -26, 0.0, -0.0,
                          1e-40, np.nan], np.float32))


def test_f32_to_f16_random(orc):
    g = np.random.default_rng(1)
    x = g.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    _check(orc, x)
