"""Decision-aware comparison of a binary32 decode step with the plain binary64 reference.

The fixed-order binary32 specification (oracle/stepq_oracle.c) and the GPU kernels compute one
evaluation order of the step; ``oracle/plain.py`` computes the step as the method states it, in
binary64.  Their real-valued results agree to binary32 rounding error, but every integer decision
(a binary16 row or column factor, a first or final code, a binary16 pivot value) is a rounding of
such a value, so the two can decide differently where the value lies near a rounding boundary.

``check_step`` replays one step of one tile in binary64 from the same stored state and walks the
decisions in the method's order.  At each decision the binary32 side's choice must equal the
binary64 rounding, or be the adjacent value with the binary64 value within the binary32 error
bound of the boundary between the two; the replay then continues with the binary32 side's choice
(teacher forcing), so one near-tie does not cascade.  Readouts must lie within their own bound.

Error bounds (unit roundoff u = 2^-24, gamma(n) = n u / (1 - n u); every bound uses the binary64
values in place of the exact ones, whose difference is far below these bounds):
  key projection u_j   the specification's dot is one fma chain over each block of 32 rows (the
                       first term a rounded product), then a pairwise tree over the d_k / 32
                       block sums, with the row coefficient k_i r_i rounded once: each term
                       sees at most DOT_DEPTH roundings, so |u32 - u| <= gamma(DOT_DEPTH)
                       sum_l |k_l S_hat_lj| (one more for the decay-first coefficient
                       k_i (a_i r_i)).
  error e              e = v - a_i u (one fma) or v - u: |e32 - e| <= u|e| + |a_i| |u32 - u|.
  state S_ij           the specification keeps S = M_i T_ij with M = fl(a_i r_i),
                       K = fl(fl(beta k_i) / M), T = fma(K, e32, X): M T = (a_i S_hat (1 + d1)
                       + beta k_i e32 (1 + d2)(1 + d3))(1 + d5), so |S32 - S| <= gamma(2)
                       |a_i S_hat| + |beta k_i| (gamma(4)|e| + (1 + gamma(3))|e32 - e|).  Call it
                       B_ij (S32 being the exact product M_i T_ij).
  readout o_j          dot of (q_i M_i rounded) with T: gamma(DOT_DEPTH) sum_i |q_i S_ij| +
                       sum_i |q_i| B_ij.
  row factor r_i       tree over d_v columns of |T| (ROW_DEPTH levels), times |M_i|, exact 1/d_v,
                       + 1e-8f, times the rounded 1/den (den's own binary32 rounding: ROW_DEPTH +
                       3 roundings): r rel. gamma(ROW_DEPTH + 8) + sum_j B_ij / (d_v den_i).
  y = T * (M_i/r_hat)  |y32 - S/r_hat| <= B / r_hat + gamma(3) |S / r_hat|.
  c0_j                 max over rows of (|y| * (1/qmax)) rounded twice more: per candidate
                       |.| <= (B/r_hat + gamma(5)|S/r_hat|) / qmax.
  first codes          t0 = y * (1/c0) exact product: |t0_32 - t0| <= (B/r_hat)/c0 + |t0|
                       (gamma(4) + 2 dc0/c0) (1 + 2 dc0/c0).
  refit sums           W = omega r_hat^2 (2 roundings), a = W z0 (1), num = dot(a, y),
                       sq = dot(a, z0) (DOT_DEPTH - 1 more); every term is >= 0 (z0 and y share
                       their sign), so num, sq carry relative errors gamma(DOT_DEPTH + 2) plus
                       sum_i W_i |z0_ij| |y32 - y| / num; c1 = num / sq adds u.
  final codes          t = y * (1/c_hat): |t32 - t| <= (B/r_hat)/c_hat + gamma(5)|t|.
  pivot values         |S32 - S| <= B_ij.
Every bound is multiplied by SAFETY.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from oracle import codec, plain

U = 2.0 ** -24
DOT_DEPTH = 35      # 32 (one chain per block of 32 rows) + log2(128 / 32) + 1 (coefficient)
ROW_DEPTH = 7       # pairwise tree over 128 values
SAFETY = 1.25
EPS_SPEC = float(np.float32(1e-8))   # the specification's 1e-8f


def gam(n):
    return n * U / (1.0 - n * U)


class PlainMismatch(AssertionError):
    pass


@dataclass
class PlainStats:
    steps: int = 0
    forced: dict = field(default_factory=lambda: dict(r=0, c=0, z0=0, z=0, h=0))
    worst_ratio: float = 0.0       # max over forced decisions of distance / bound (<= 1)
    z_beyond_1e5: int = 0          # forced final codes whose binary64 value is > 1e-5 from .5
    z_max_dist: float = 0.0        # max distance of a forced final code's value from .5
    worst_readout_rel: float = 0.0
    worst_readout_ratio: float = 0.0

    def merge(self, o: "PlainStats"):
        self.steps += o.steps
        for k in self.forced:
            self.forced[k] += o.forced[k]
        self.worst_ratio = max(self.worst_ratio, o.worst_ratio)
        self.z_beyond_1e5 += o.z_beyond_1e5
        self.z_max_dist = max(self.z_max_dist, o.z_max_dist)
        self.worst_readout_rel = max(self.worst_readout_rel, o.worst_readout_rel)
        self.worst_readout_ratio = max(self.worst_readout_ratio, o.worst_readout_ratio)

    def summary(self) -> str:
        f = self.forced
        return (f"plain: {self.steps} tile-steps, forced decisions r {f['r']} c {f['c']} "
                f"z0 {f['z0']} z {f['z']} h {f['h']} (worst distance/bound {self.worst_ratio:.2f};"
                f" final codes beyond 1e-5 of .5: {self.z_beyond_1e5}, max {self.z_max_dist:.2e}),"
                f" readout rel L2 <= {self.worst_readout_rel:.1e}")


def _f16_ordered(h):
    """binary16 bit patterns -> integers in the order of their values (adjacent values differ
    by 1; +0 and -0 both map to 0)."""
    h = np.asarray(h, np.int64)
    return np.where(h & 0x8000, -(h & 0x7FFF), h)


def _f16_from_ordered(o):
    """Inverse of _f16_ordered (0 -> +0)."""
    o = np.asarray(o, np.int64)
    return np.where(o < 0, 0x8000 | (-o), o).astype(np.uint16)


def _f16_interval(h):
    """The reals that round to binary16 value h (round-half-even; ties counted in): the
    midpoints with its two neighbours.  Past the largest finite value the threshold of
    overflow (65520) stands in for the midpoint with infinity."""
    o = _f16_ordered(h)
    v = plain.f16(np.asarray(h, np.uint16)).astype(np.float64)
    lo_n = plain.f16(_f16_from_ordered(np.maximum(o - 1, -0x7BFF))).astype(np.float64)
    hi_n = plain.f16(_f16_from_ordered(np.minimum(o + 1, 0x7BFF))).astype(np.float64)
    lo = np.where(o <= -0x7BFF, -65520.0, 0.5 * (v + lo_n))
    hi = np.where(o >= 0x7BFF, 65520.0, 0.5 * (v + hi_n))
    return lo, hi


def _check_f16(kind, x64, h_side, bound, st: PlainStats, where):
    """binary16 decision: h_side (bit patterns) against fl16(x64).  A different value passes when
    the binary64 value lies within the binary32 error bound of the reals that round to the
    binary32 side's value (for neighbours: of the boundary between the two; where the bound
    spans several binary16 steps, as for an entry left small by cancellation, several values
    are consistent with it)."""
    h_plain = plain.fl16(x64).view(np.uint16)
    h_side = np.asarray(h_side, np.uint16)
    diff = h_plain != h_side
    # +0 / -0 are the same decision
    diff &= ~((h_plain & 0x7FFF) == 0) | ~((h_side & 0x7FFF) == 0)
    if not diff.any():
        return
    idx = np.nonzero(diff)
    x = np.asarray(x64, np.float64)[idx]
    bd = np.asarray(bound, np.float64)[idx] if np.ndim(bound) else np.full(x.shape, bound)
    lo, hi = _f16_interval(h_side[idx])
    dist = np.maximum(0.0, np.maximum(lo - x, x - hi))
    ok = dist <= bd + 1e-12 * np.abs(x)
    if not ok.all():
        k = int(np.argmin(ok))
        raise PlainMismatch(
            f"{where}: {kind} decision differs beyond the binary32 error bound at "
            f"{tuple(int(t[k]) for t in idx)}: binary64 {x[k]!r} -> {plain.f16(h_plain[idx][k])!r}, "
            f"binary32 side {plain.f16(h_side[idx][k])!r}, distance {dist[k]:.3e} > bound {bd[k]:.3e}")
    st.forced[kind] += int(diff.sum())
    st.worst_ratio = max(st.worst_ratio, float(np.max(dist / np.maximum(bd, 1e-300))))


def _check_codes(kind, t64, z_side, qm, bound, st: PlainStats, where):
    """Integer decision: z_side against clip(rne(t64), +-qmax)."""
    z_plain = plain.round_codes(t64, qm)
    z_side = np.asarray(z_side, np.float64)
    diff = z_plain != z_side
    if not diff.any():
        return
    idx = np.nonzero(diff)
    mid = 0.5 * (z_plain[idx] + z_side[idx])
    t = t64[idx]
    dist = np.abs(t - mid)
    bd = bound[idx]
    ok = (np.abs(z_plain[idx] - z_side[idx]) == 1) & (dist <= bd + 1e-12 * np.abs(t))
    if not ok.all():
        k = int(np.argmin(ok))
        raise PlainMismatch(
            f"{where}: {kind} differs away from a rounding boundary at "
            f"{(int(idx[0][k]), int(idx[1][k]))}: binary64 value {t[k]!r} -> {z_plain[idx][k]:.0f}, "
            f"binary32 side {z_side[idx][k]:.0f}, distance from .5 {dist[k]:.3e} > bound {bd[k]:.3e}")
    st.forced[kind] += int(diff.sum())
    st.worst_ratio = max(st.worst_ratio, float(np.max(dist / np.maximum(bd, 1e-300))))
    if kind == "z":
        st.z_beyond_1e5 += int(np.sum(dist > 1e-5))
        st.z_max_dist = max(st.z_max_dist, float(dist.max()))


def check_step(bits, pivot, omega, order, seg_before, seg_after, out_side, z0_side, q, k, v, a,
               beta, where="", st: PlainStats | None = None, c0_side=None) -> PlainStats:
    """One decode step of one tile: seg_before (stored state), the binary32 side's readout
    out_side and result seg_after, and the side's first codes z0_side (the one decision the
    packed state does not show).  Raises PlainMismatch on any difference the bounds above do not
    explain; returns the updated statistics."""
    st = PlainStats() if st is None else st
    bits = np.asarray(bits, np.int64)
    piv = np.asarray(pivot).astype(bool)
    om = np.asarray(omega, np.float64)
    dk = bits.size
    dv = dk
    qm = np.where(piv, 0.0, plain.qmax(bits))
    z, r16, c16, h16 = codec.unpack(seg_before, bits, piv, dv)
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    a = np.asarray(a, np.float64) * np.ones(dk)
    beta = float(beta)

    # ---- the step in binary64 (plain reference) and the state's error bound B
    S_hat = plain.decode(r16, c16, z, h16, piv)
    S = plain.update(S_hat, k, v, a, beta, order)
    o = plain.readout(S, q)
    kS = np.abs(k)[:, None] * np.abs(S_hat)
    if order == plain.DELTA_FIRST:
        u = k @ S_hat
        e = v[None, :] - a[:, None] * u[None, :]
        eps_u = gam(DOT_DEPTH) * kS.sum(axis=0)
        eps_e = U * np.abs(e) + np.abs(a)[:, None] * eps_u[None, :]
    else:
        u = (k * a) @ S_hat
        e = np.broadcast_to(v - u, (dk, dv))
        eps_u = gam(DOT_DEPTH + 1) * (np.abs(a)[:, None] * kS).sum(axis=0)
        eps_e = U * np.abs(e) + eps_u[None, :]
    bk = np.abs(beta * k)[:, None]
    B = gam(2) * np.abs(a[:, None] * S_hat) + bk * (gam(4) * np.abs(e) + (1 + gam(3)) * eps_e)
    B = SAFETY * B + 2.0 ** -140

    # ---- readout
    out_side = np.asarray(out_side, np.float64)
    bo = SAFETY * (gam(DOT_DEPTH) * (np.abs(q)[:, None] * np.abs(S)).sum(axis=0)
                   + (1 + gam(DOT_DEPTH)) * (np.abs(q)[:, None] * B).sum(axis=0))
    err = np.abs(out_side - o)
    if np.any(err > bo):
        j = int(np.argmax(err / bo))
        raise PlainMismatch(f"{where}: readout column {j}: binary32 {out_side[j]!r} binary64 "
                            f"{o[j]!r}, error {err[j]:.3e} > bound {bo[j]:.3e}")
    no = np.linalg.norm(o)
    rel = float(np.linalg.norm(out_side - o) / (no if no > 0 else 1.0))
    st.worst_readout_rel = max(st.worst_readout_rel, rel)
    st.worst_readout_ratio = max(st.worst_readout_ratio, float(np.max(err / bo)))

    z_s, r16_s, c16_s, h16_s = codec.unpack(seg_after, bits, piv, dv)

    # ---- pivot rows: binary16 of the updated state
    if piv.any():
        _check_f16("h", S[piv], h16_s[piv], B[piv], st, where + " pivot rows")
    if piv.all():
        st.steps += 1
        return st

    # ---- row factors
    den = plain.row_den(om)
    r64 = plain.row_factor(S, den)
    absS = np.abs(S).sum(axis=1)
    br = SAFETY * (r64 * gam(ROW_DEPTH + 8)
                   + ((gam(ROW_DEPTH + 1) * absS + (1 + gam(ROW_DEPTH + 1)) * B.sum(axis=1)) / dv
                      + abs(EPS_SPEC - plain.EPS_ROW)) / den * (1 + gam(3)))
    q_rows = ~piv
    _check_f16("r", r64[q_rows], r16_s[q_rows], br[q_rows], st, where + " row factors")
    r_hat = np.where(piv, 0.0, plain.f16(r16_s))            # teacher-forced
    live = plain.live_rows(piv, r_hat)
    rl = np.where(live, r_hat, 1.0)

    # ---- first column factors and first codes
    y = S / rl[:, None]
    by = B / rl[:, None] + gam(3) * np.abs(y)
    c0 = plain.column_init(S, r_hat, np.where(piv, 1.0, qm), live)
    cand = np.where(live[:, None], (by + gam(2) * np.abs(y)) / np.where(piv, 1.0, qm)[:, None], 0)
    bc0 = SAFETY * cand.max(axis=0)
    if c0_side is not None:
        d = np.abs(np.asarray(c0_side, np.float64) - c0)
        if np.any(d > bc0 + 1e-300):
            j = int(np.argmax(d - bc0))
            raise PlainMismatch(f"{where}: first column factor {j}: binary32 {c0_side[j]!r} "
                                f"binary64 {c0[j]!r} beyond bound {bc0[j]:.3e}")
    c0s = np.where(c0 > 0, c0, 1.0)
    rc = np.where(c0 > 0, bc0 / c0s, 0.0)
    t0 = plain.scaled(S, r_hat, c0, live)
    bt0 = SAFETY * ((B / rl[:, None]) / c0s[None, :] + np.abs(t0) * (gam(4) + 2 * rc[None, :])) \
        * (1 + 2 * rc[None, :])
    m0 = live[:, None] & (c0 > 0)[None, :]
    z0_side = np.asarray(z0_side, np.float64)
    if np.any(z0_side[~m0] != 0):
        raise PlainMismatch(f"{where}: nonzero first code on a dead or pivot row or column")
    _check_codes("z0", np.where(m0, t0, 0.0), np.where(m0, z0_side, 0.0),
                 np.where(piv, 0.0, qm), np.where(m0, bt0, 0.0), st, where + " first codes")
    z0 = z0_side                                              # teacher-forced

    # ---- least-squares refit of the column factors
    c1 = plain.refit(S, r_hat, z0, om, c0, live)
    W = np.where(live, om * r_hat * r_hat, 0.0)
    num = (W[:, None] * z0 * y).sum(axis=0)
    sq = (W[:, None] * z0 * z0).sum(axis=0)
    dnum = (W[:, None] * np.abs(z0) * by).sum(axis=0)
    ok_sq = sq > 0
    rel_c1 = U + 2 * gam(DOT_DEPTH + 2) + dnum / np.where(num > 0, num, 1.0)
    bc1 = SAFETY * np.where(ok_sq, np.abs(c1) * rel_c1 * (1 + gam(4)), bc0)
    _check_f16("c", c1, c16_s, bc1, st, where + " column factors")
    c_hat = plain.f16(c16_s)                                  # teacher-forced

    # ---- final codes
    t = plain.scaled(S, r_hat, c_hat, live)
    cs = np.where(c_hat != 0, c_hat, 1.0)
    bt = SAFETY * ((B / rl[:, None]) / cs[None, :] + gam(5) * np.abs(t))
    m = live[:, None] & (c_hat != 0)[None, :]
    z_s = np.asarray(z_s, np.float64)
    if np.any(z_s[~m] != 0):
        raise PlainMismatch(f"{where}: nonzero code on a dead or pivot row or column")
    _check_codes("z", np.where(m, t, 0.0), np.where(m, z_s, 0.0), np.where(piv, 0.0, qm),
                 np.where(m, bt, 0.0), st, where + " codes")
    st.steps += 1
    return st


def check_encode(bits, pivot, omega, S32, seg_after, z0_side, where="",
                 st: PlainStats | None = None) -> PlainStats:
    """Entering an fp32 state: the requantization decisions of seg_after against the plain
    reference on the given binary32 state (which both sides read exactly, B = 0)."""
    st = PlainStats() if st is None else st
    bits = np.asarray(bits, np.int64)
    piv = np.asarray(pivot).astype(bool)
    om = np.asarray(omega, np.float64)
    dk = dv = bits.size
    qm = np.where(piv, 0.0, plain.qmax(bits))
    S = np.asarray(S32, np.float64)
    z_s, r16_s, c16_s, h16_s = codec.unpack(seg_after, bits, piv, dv)
    if piv.any():
        _check_f16("h", S[piv], h16_s[piv], np.zeros(int(piv.sum()) * dv).reshape(-1, dv) + 2.0**-140,
                   st, where + " pivot rows")
    if piv.all():
        st.steps += 1
        return st
    den = plain.row_den(om)
    r64 = plain.row_factor(S, den)
    br = SAFETY * (r64 * gam(ROW_DEPTH + 8) + (gam(ROW_DEPTH + 1) * np.abs(S).sum(axis=1) / dv
                                               + abs(EPS_SPEC - plain.EPS_ROW)) / den)
    _check_f16("r", r64[~piv], r16_s[~piv], br[~piv], st, where + " row factors")
    r_hat = np.where(piv, 0.0, plain.f16(r16_s))
    live = plain.live_rows(piv, r_hat)
    rl = np.where(live, r_hat, 1.0)
    y = S / rl[:, None]
    c0 = plain.column_init(S, r_hat, np.where(piv, 1.0, qm), live)
    cand = np.where(live[:, None], gam(5) * np.abs(y) / np.where(piv, 1.0, qm)[:, None], 0)
    bc0 = SAFETY * cand.max(axis=0)
    c0s = np.where(c0 > 0, c0, 1.0)
    rc = np.where(c0 > 0, bc0 / c0s, 0.0)
    t0 = plain.scaled(S, r_hat, c0, live)
    bt0 = SAFETY * np.abs(t0) * (gam(4) + 2 * rc[None, :]) * (1 + 2 * rc[None, :])
    m0 = live[:, None] & (c0 > 0)[None, :]
    z0_side = np.asarray(z0_side, np.float64)
    _check_codes("z0", np.where(m0, t0, 0.0), np.where(m0, z0_side, 0.0),
                 np.where(piv, 0.0, qm), np.where(m0, bt0, 0.0), st, where + " first codes")
    z0 = z0_side
    c1 = plain.refit(S, r_hat, z0, om, c0, live)
    W = np.where(live, om * r_hat * r_hat, 0.0)
    num = (W[:, None] * z0 * y).sum(axis=0)
    dnum = (W[:, None] * np.abs(z0) * gam(3) * np.abs(y)).sum(axis=0)
    sq = (W[:, None] * z0 * z0).sum(axis=0)
    rel_c1 = U + 2 * gam(DOT_DEPTH + 2) + dnum / np.where(num > 0, num, 1.0)
    bc1 = SAFETY * np.where(sq > 0, np.abs(c1) * rel_c1 * (1 + gam(4)), bc0)
    _check_f16("c", c1, c16_s, bc1, st, where + " column factors")
    c_hat = plain.f16(c16_s)
    t = plain.scaled(S, r_hat, c_hat, live)
    bt = SAFETY * gam(5) * np.abs(t)
    m = live[:, None] & (c_hat != 0)[None, :]
    z_s = np.asarray(z_s, np.float64)
    _check_codes("z", np.where(m, t, 0.0), np.where(m, z_s, 0.0), np.where(piv, 0.0, qm),
                 np.where(m, bt, 0.0), st, where + " codes")
    st.steps += 1
    return st
