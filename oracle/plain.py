"""Plain binary64 reference of the STEPQuant decode step: the step as the method states it.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may use ``oracle/``; the product never does.

This module is the definition the fixed-order binary32 specification (``stepq_oracle.c``) and
the GPU kernels are checked against.  It computes every quantity in binary64 in the order the
method describes it, with matrix products and explicit formulas, and has no lane layout, no
blocking and no fused-multiply-add structure.  Integer decisions (binary16 factors, codes) are
taken by rounding the binary64 value; the checker in ``tests/plainparity.py`` accepts a different
decision by the binary32 specification only where the binary64 value lies within the binary32
error bound of the rounding boundary.

Page: "STEPQuant" paper digest (vibe-research silicon-writer readme).
  Background ("linear attention only changes the memory bill", "why plain INT8 is still not
  stable"): S_t = A_t S_{t-1} + beta_t k_t v_t^T, A_t holds the retention gate and the delta
  update, o_t = S_t^T q_t.
  Method 3 ("Key-Row-Aware Dual-Axis Fitting"): X_hat = r_i c_j z_ij, r_i from the row's mean
  magnitude with finer steps for high-omega rows, c_j an omega-weighted mean-squared-error fit
  with r fixed, low-bit integer codes z.
  Method 4 ("the execution path of each decode step"): reconstruct, update, read out before
  requantization, refit r and c, pack codes, scales and FP16 pivots back.
Readings where the pages leave the step open (the same as the binary32 specification's):
  A_t = Diag(a)(I - beta k k^T) (order 0) or (I - beta k k^T) Diag(a) (order 1);
  r_i = (mean_j |S_ij| + 1e-8) / (1 + omega_i / mean_i omega) (pivot rows take no factor);
  c0_j = max_i |S_ij / r_hat_i| / qmax_i over live rows;  z0 = rne(S / (r_hat c0));
  c1_j = argmin_c sum_i omega_i (S_ij - r_hat_i c z0_ij)^2 (normal equation);
  z = clip(rne(S / (r_hat c_hat)), -qmax, qmax), qmax = 2^(b-1) - 1, half-way cases to even;
  r_hat, c_hat and pivot values are binary16 (round to nearest even); a row or column whose
  binary16 factor is 0 is dead (all its codes 0).
"""
from __future__ import annotations

import numpy as np

DELTA_FIRST, DECAY_FIRST = 0, 1
EPS_ROW = 1e-8


def fl16(x) -> np.ndarray:
    """binary64 -> binary16, round to nearest even (overflow to infinity)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float64).astype(np.float16)


def f16(h) -> np.ndarray:
    """binary16 bit patterns -> binary64 values."""
    return np.asarray(h, np.uint16).view(np.float16).astype(np.float64)


def qmax(bits) -> np.ndarray:
    return (2.0 ** (np.asarray(bits, np.float64) - 1.0)) - 1.0


def row_den(omega) -> np.ndarray:
    """1 + omega_i / mean(omega) over the head's rows; 1 if the mean is 0."""
    om = np.asarray(omega, np.float64)
    m = om.mean()
    return 1.0 + om / m if m > 0 else np.ones_like(om)


def decode(r16, c16, z, h16, pivot) -> np.ndarray:
    """S_hat_ij = r_hat_i c_hat_j z_ij; pivot rows hold their binary16 values (Method 3,
    Method 4 step 1)."""
    piv = np.asarray(pivot).astype(bool)
    S = f16(r16)[:, None] * f16(c16)[None, :] * np.asarray(z, np.float64)
    S[piv] = f16(h16)[piv]
    return S


def gate_matrix(k, a, beta, order=DELTA_FIRST) -> np.ndarray:
    """A_t = Diag(a)(I - beta k k^T), or (I - beta k k^T) Diag(a) for order 1 (Background)."""
    k = np.asarray(k, np.float64)
    a = np.asarray(a, np.float64) * np.ones_like(k)
    P = np.eye(k.size) - float(beta) * np.outer(k, k)
    return np.diag(a) @ P if order == DELTA_FIRST else P @ np.diag(a)


def update(S_hat, k, v, a, beta, order=DELTA_FIRST) -> np.ndarray:
    """S_t = A_t S_hat + beta k v^T (Background)."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    return gate_matrix(k, a, beta, order) @ S_hat + float(beta) * np.outer(k, v)


def readout(S, q) -> np.ndarray:
    """o_t = S_t^T q_t, from the updated float state (Method 4: before requantization)."""
    return S.T @ np.asarray(q, np.float64)


def row_factor(S, den) -> np.ndarray:
    """r_i = (mean_j |S_ij| + 1e-8) / den_i (Method 3: grows with the row's mean magnitude,
    smaller steps for high-impact rows)."""
    return (np.abs(S).mean(axis=1) + EPS_ROW) / np.asarray(den, np.float64)


def live_rows(pivot, r_hat) -> np.ndarray:
    return ~np.asarray(pivot).astype(bool) & (np.asarray(r_hat, np.float64) != 0.0)


def column_init(S, r_hat, qm, live) -> np.ndarray:
    """c0_j = max over live rows of |S_ij / r_hat_i| / qmax_i (0 for an all-dead column)."""
    if not live.any():
        return np.zeros(S.shape[1])
    x = np.abs(S[live] / r_hat[live, None]) / qm[live, None]
    return x.max(axis=0)


def scaled(S, r_hat, c, live) -> np.ndarray:
    """t_ij = S_ij / (r_hat_i c_j) on live rows and columns (c_j != 0), 0 elsewhere: the value
    that the quantizer rounds."""
    cl = c != 0.0
    m = live[:, None] & cl[None, :]
    grid = np.where(live, r_hat, 1.0)[:, None] * np.where(cl, c, 1.0)[None, :]
    return np.where(m, S / grid, 0.0)


def round_codes(t, qm) -> np.ndarray:
    """Symmetric round half to even, clipped to +-qmax."""
    return np.clip(np.rint(t), -qm[:, None], qm[:, None])


def refit(S, r_hat, z0, omega, c0, live) -> np.ndarray:
    """c1_j = argmin_c sum_i omega_i (S_ij - r_hat_i c z0_ij)^2 with z0 fixed (Method 3's
    omega-weighted fit with r fixed), from its normal equation
    c1 = sum_i omega_i p_ij S_ij / sum_i omega_i p_ij^2, p = r_hat z0; c1 = c0 where the
    denominator is 0."""
    om = np.where(live, np.asarray(omega, np.float64), 0.0)
    p = r_hat[:, None] * np.asarray(z0, np.float64)
    num = (om[:, None] * p * S).sum(axis=0)
    den = (om[:, None] * p * p).sum(axis=0)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), c0)


def requantize(S, bits, pivot, omega):
    """Steps after the readout (Method 4 steps 4-5): row factors, first column factors, first
    codes, least-squares column refit, final codes.  Returns a dict of every intermediate:
    r (binary64), r16, c0, t0, z0, c1, c16, t, z and h16 (pivot rows)."""
    piv = np.asarray(pivot).astype(bool)
    qm = qmax(bits)
    r = row_factor(S, row_den(omega))
    r16 = np.where(piv, np.float16(0), fl16(r)).astype(np.float16)
    r_hat = r16.astype(np.float64)
    live = live_rows(piv, r_hat)
    c0 = column_init(S, r_hat, qm, live)
    t0 = scaled(S, r_hat, c0, live)
    z0 = round_codes(t0, qm)
    c1 = refit(S, r_hat, z0, omega, c0, live)
    c16 = fl16(c1)
    c_hat = c16.astype(np.float64)
    t = scaled(S, r_hat, c_hat, live)
    z = round_codes(t, qm)
    h16 = np.where(piv[:, None], fl16(S), np.float16(0)).astype(np.float16)
    return dict(r=r, r16=r16, c0=c0, t0=t0, z0=z0, c1=c1, c16=c16, t=t, z=z, h16=h16)


def step(fields, bits, pivot, omega, q, k, v, a, beta, order=DELTA_FIRST):
    """One decode step of one tile.  fields = (z, r16, c16, h16) of the stored state (bit
    patterns for the binary16 arrays).  Returns (o, S, requantize(S) dict)."""
    z, r16, c16, h16 = fields
    S_hat = decode(r16, c16, z, h16, pivot)
    S = update(S_hat, k, v, a, beta, order)
    o = readout(S, q)
    return o, S, requantize(S, bits, pivot, omega)


def encode(S, bits, pivot, omega):
    """Entering an fp32 state: the requantization alone."""
    return requantize(np.asarray(S, np.float64), bits, pivot, omega)
