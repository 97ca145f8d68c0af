"""Pins for the oracle's requantizer (Method 3, dual-axis fit) against closed forms and library
routines: the row-factor formula, the omega-weighted least-squares column refit (NumPy lstsq),
the half-step error bound, code range, FP16 pivots (NumPy binary16), dead rows and columns, and
the bits/value accounting."""
import numpy as np
import pytest

from layout_ref import read_codes, read_f16, seg_fields


def _structured_state(g, dk, dv):
    rho = np.exp(g.standard_normal(dk))
    gam = np.exp(g.standard_normal(dv))
    return (rho[:, None] * g.standard_normal((dk, dv)) * gam[None, :]).astype(np.float32)


def _head(g, dk, dv, kda=True, npiv=2):
    if kda:
        bits = g.choice([2, 4, 6, 8], size=dk).astype(np.int8)
    else:
        bits = np.full(dk, int(g.choice([2, 4, 6, 8])), np.int8)
    piv = np.zeros(dk, np.uint8)
    if npiv:
        piv[g.choice(dk, npiv, replace=False)] = 1
    omega = g.exponential(1.0, dk).astype(np.float32)
    return bits, piv, omega


def _decode64(seg, bits, piv, dv):
    f = seg_fields(bits, piv, dv)
    r = read_f16(seg, f["off_r"], len(bits)).view(np.float16).astype(np.float64)
    c = read_f16(seg, f["off_c"], dv).view(np.float16).astype(np.float64)
    z = read_codes(seg, bits, piv, dv)
    return r, c, z


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("dk", [64, 128])
def test_requantizer_invariants(orc, seed, dk):
    g = np.random.default_rng(100 + seed)
    dv = dk
    bits, piv, omega = _head(g, dk, dv, kda=seed % 2 == 0, npiv=seed % 3)
    S = _structured_state(g, dk, dv)
    seg, pre, flags = orc.Head(bits, piv, omega, dv).encode(S, want_pre=True)
    assert flags == 0
    r, c, z = _decode64(seg, bits, piv, dv)
    live = piv == 0
    qmax = (1 << (bits.astype(np.int64) - 1)) - 1

    # codes in range, pivot rows hold no codes
    assert np.all(np.abs(z) <= qmax[:, None])
    assert np.all(z[~live] == 0)

    # row factor: r_i = (mean_j |S_ij| + 1e-8) / (1 + omega_i / mean omega), in binary16
    S64 = S.astype(np.float64)
    r_ref = (np.mean(np.abs(S64), axis=1) + 1e-8) / (1 + omega / np.mean(omega.astype(np.float64)))
    r_ref16 = r_ref.astype(np.float16).astype(np.float64)
    ulp = np.spacing(r_ref.astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(r[live] - r_ref16[live]) <= ulp[live])
    assert np.mean(r[live] == r_ref16[live]) >= 0.98

    # column refit: c1_j = argmin_c sum_i omega_i (S_ij - r_i c z0_ij)^2 with z0 from
    # c0_j = max_i |S_ij / r_i| / qmax_i, solved by weighted least squares (NumPy lstsq)
    y = np.where(live[:, None], S64 / np.where(r > 0, r, 1)[:, None], 0.0)
    y[r == 0] = 0.0
    c0 = np.max(np.abs(y) / np.where(live, qmax, 1)[:, None], axis=0)
    z0 = np.rint(y / np.where(c0 > 0, c0, 1)[None, :])
    agree = 0
    for j in range(dv):
        sw = np.sqrt(omega.astype(np.float64)) * live
        A = (sw * r * z0[:, j])[:, None]
        sol = np.linalg.lstsq(A, sw * S64[:, j], rcond=None)[0][0] if np.any(A) else c0[j]
        c16 = np.float16(sol).astype(np.float64)
        assert abs(c[j] - c16) <= float(np.spacing(np.float16(sol))) * 1.01, (j, c[j], sol)
        agree += c[j] == c16
    assert agree >= 0.95 * dv

    # half-step bound on every unclipped entry, with the refitted factors
    step = r[:, None] * c[None, :]
    unclipped = live[:, None] & (np.abs(pre) <= qmax[:, None] + 0.5)
    err = np.abs(S64 - step * z)
    assert np.all(err[unclipped] <= 0.5 * step[unclipped] * (1 + 1e-5) + 1e-30)

    # FP16 pivots are the binary16 rounding of the state, bit for bit
    f = seg_fields(bits, piv, dv)
    if f["npiv"]:
        got = read_f16(seg, f["off_piv"], f["npiv"] * dv).reshape(f["npiv"], dv)
        assert np.array_equal(got, S[piv == 1].astype(np.float16).view(np.uint16))


def test_dead_rows_and_columns(orc):
    g = np.random.default_rng(9)
    dk = dv = 64
    bits, piv, omega = np.full(dk, 6, np.int8), np.zeros(dk, np.uint8), np.ones(dk, np.float32)
    S = g.standard_normal((dk, dv)).astype(np.float32)
    S[5, :] = 0.0
    S[:, 9] = 0.0
    seg = orc.Head(bits, piv, omega).encode(S)
    r, c, z = _decode64(seg, bits, piv, dv)
    assert r[5] == 0.0 and np.all(z[5] == 0)        # 1e-8/den rounds to zero in binary16
    assert c[9] == 0.0 and np.all(z[:, 9] == 0)
    S2, _, _, _ = orc.Head(bits, piv, omega).unpack(seg)
    assert np.all(S2[5] == 0) and np.all(S2[:, 9] == 0)
    seg0 = orc.Head(bits, piv, omega).encode(np.zeros((dk, dv), np.float32))
    S0, _, _, _ = orc.Head(bits, piv, omega).unpack(seg0)
    assert np.all(S0 == 0)


def test_all_pivot_head_is_raw_fp16(orc):
    g = np.random.default_rng(11)
    dk = dv = 128
    S = g.standard_normal((dk, dv)).astype(np.float32)
    h = orc.Head(np.full(dk, 6, np.int8), np.ones(dk, np.uint8), np.ones(dk, np.float32))
    seg = h.encode(S)
    assert np.array_equal(seg.view(np.uint16), S.astype(np.float16).view(np.uint16).ravel())


def test_flags_on_overflow_and_nonfinite(orc):
    dk = dv = 64
    bits, omega = np.full(dk, 4, np.int8), np.ones(dk, np.float32)
    S = np.ones((dk, dv), np.float32)
    S[3, 3] = np.inf
    _, _, fl = orc.Head(bits, np.zeros(dk, np.uint8), omega).encode(S, want_pre=True)
    assert fl & orc.FLAG_NONFINITE
    S = np.full((dk, dv), 1e6, np.float32)       # row factor 1e6 > 65504
    _, _, fl = orc.Head(bits, np.zeros(dk, np.uint8), omega).encode(S, want_pre=True)
    assert fl & orc.FLAG_SCALE_OVF
    piv = np.zeros(dk, np.uint8)
    piv[0] = 1
    S = np.ones((dk, dv), np.float32)
    S[0, 0] = 1e5
    _, _, fl = orc.Head(bits, piv, omega).encode(S, want_pre=True)
    assert fl & orc.FLAG_PIVOT_OVF


def closed_form_bits(bits, piv, dv):
    """Payload bits of one head: codes + FP16 pivot rows + FP16 row/column factors."""
    live = piv == 0
    code = dv * int(np.sum(bits[live].astype(np.int64)))
    pivots = 16 * dv * int(np.sum(~live))
    scales = 0 if not live.any() else 16 * (len(bits) + dv)
    return code + pivots + scales


@pytest.mark.parametrize("seed", range(4))
def test_bits_per_value_accounting(orc, seed):
    g = np.random.default_rng(seed)
    dk = dv = 128
    bits, piv, omega = _head(g, dk, dv, kda=seed % 2 == 0, npiv=seed)
    f = seg_fields(bits, piv, dv)
    # payload fields of the layout: words hold the lane streams (padding < 32 bits per lane)
    G = dv // 64
    lane_bits = G * int(np.sum(bits[piv == 0].astype(np.int64)))
    assert 8 * (f["off_piv"]) - 64 * lane_bits < 64 * 32
    payload = 64 * lane_bits + 8 * (f["off_c"] - f["off_piv"]) + (0 if f["allpiv"] else 16 * dv)
    assert payload == closed_form_bits(bits, piv, dv)
    assert 8 * orc.Head(bits, piv, omega, dv).seg_bytes >= payload
