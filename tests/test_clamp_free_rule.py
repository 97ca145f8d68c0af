"""The GDN tiles leave out the final clamp when every column passes
fma(ymax_j, ic_j, kMagic) <= kMagic + qmax, ymax_j = max_i |y_ij|.  The claim behind it: the
offset-domain rounding fma(y, ic, kMagic) (round to nearest even, kMagic = 1.5 * 2^23) is monotone
in y and symmetric about kMagic, so every |y| <= ymax then rounds to a code within +-qmax.  Checked
here with an exact emulation of that fma (the binary32 product is exact in binary64; one
rounding: the exact product rounded half to even to an integer, which is what binary32 spacing 1
around kMagic gives), over random columns and over ties placed exactly at the boundary."""
import numpy as np

M = np.float32(12582912.0)


def fma_magic(y, ic):
    # y * ic is exact in binary64 (24 + 24 bits); binary32 spacing is 1 on [2^23, 2^24), so the
    # one rounding of fma(y, ic, kMagic) is kMagic + (y * ic rounded half to even to an integer)
    # while |y * ic| < 2^22 (returned as its exact binary64 value)
    p = np.asarray(y, np.float32).astype(np.float64) * np.float64(np.float32(ic))
    assert np.all(np.abs(p) < 2.0**22)
    return np.float64(M) + np.rint(p)


def test_column_test_implies_no_clamp():
    g = np.random.default_rng(5)
    for qm in (1, 7, 31, 127):
        for _ in range(400):
            n = 128
            y = (g.standard_normal(n) * g.lognormal(0, 2)).astype(np.float32)
            ymax = np.abs(y).max()
            # a column factor around the one that puts ymax at qmax, some passing, some not
            ic = np.float32(qm / ymax * g.uniform(0.98, 1.02))
            passes = fma_magic(ymax, ic) <= M + np.float32(qm)
            codes = fma_magic(y, ic) - np.float64(M)
            if passes:
                assert np.all(np.abs(codes) <= qm)
            # symmetry about kMagic: -y rounds to minus the code of y
            assert np.array_equal(fma_magic(-y, ic) - np.float64(M), -codes)


def test_ties_at_the_boundary_round_to_even():
    # y * ic exactly qmax + 1/2: round half to even lands on qmax + 1 for even qmax + 1 (all
    # qmax = 2^(b-1) - 1 are odd), so the test fails there and the clamp is kept
    for qm in (1, 7, 31, 127):
        y = np.float32(qm + 0.5)
        assert fma_magic(y, np.float32(1.0)) == M + np.float32(qm + 1)
        assert not fma_magic(y, np.float32(1.0)) <= M + np.float32(qm)
        assert fma_magic(np.float32(qm + 0.25), np.float32(1.0)) == M + np.float32(qm)
