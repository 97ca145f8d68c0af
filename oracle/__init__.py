"""CPU oracle for the STEPQuant packed-state decode step.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow specification that the GPU library
is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it; the product package never does, and this package imports nothing
from the product.

Two parts:

* ``stepq_oracle.c`` (loaded through ctypes): the per-tile decode step in binary32 with a fixed
  evaluation order -- dequantize, gated delta update, readout, row/column factor refit,
  requantize, pack -- plus the FP32-state step used for warm-up and drift.
* this module (NumPy, binary64): the offline inputs of the kernel -- lifetime weight L_u, row
  impact omega, pivot choice, multiple-choice dynamic programming and Lagrangian bit allocation.

Page followed throughout: "STEPQuant" paper digest (vibe-research silicon-writer readme),
Method 1 "Lifetime-aware Bit Allocation", Method 2 "Row-impact", Method 3 "Key-Row-Aware
Dual-Axis Fitting", Method 4 "the execution path of each decode step".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "stepq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

FLAG_NONFINITE = 1
FLAG_SCALE_OVF = 2
FLAG_PIVOT_OVF = 4

_CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i, l, f = ctypes.c_int, ctypes.c_long, ctypes.c_float
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f32_to_f16.argtypes = [f]
        L.orc_f16_to_f32.restype = f
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f32_to_f16_n.argtypes = [P, P, l]
        L.orc_f16_to_f32_n.argtypes = [P, P, l]
        L.orc_tree_sum.restype = f
        L.orc_tree_sum.argtypes = [P, i]
        L.orc_dot.restype = f
        L.orc_dot.argtypes = [P, P, i]
        L.orc_segment_bytes.restype = l
        L.orc_segment_bytes.argtypes = [i, i, P, P]
        L.orc_row_den.argtypes = [i, P, P]
        L.orc_unpack.restype = i
        L.orc_unpack.argtypes = [i, i, P, P, P, P, P, P, P]
        L.orc_encode.restype = i
        L.orc_encode.argtypes = [i, i, P, P, P, P, P, P, P]
        L.orc_tile_step_o.restype = i
        L.orc_tile_step_o.argtypes = [i, i, P, P, P, P, P, P, P, P, f, P, P, P, P, i]
        L.orc_encode_dbg.restype = i
        L.orc_encode_dbg.argtypes = [i, i, P, P, P, P, P, P, P, P, P]
        L.orc_tile_step_dbg.restype = i
        L.orc_tile_step_dbg.argtypes = [i, i, P, P, P, P, P, P, P, P, f, P, P, P, P, P, P, i]
        L.orc_fp32_step_o.argtypes = [i, i, P, P, P, P, P, f, P, i]
        L.orc_fp32_run_o.argtypes = [i, i, i, i, P, P, P, P, l, P, l, P, P, i]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# ----------------------------------------------------------------------------------------------
# binary16
# ----------------------------------------------------------------------------------------------

def f32_to_f16_bits(x) -> np.ndarray:
    x = _c(x, np.float32).ravel()
    h = np.empty(x.size, np.uint16)
    lib().orc_f32_to_f16_n(_p(x), _p(h), x.size)
    return h


def f16_bits_to_f32(h) -> np.ndarray:
    h = _c(h, np.uint16).ravel()
    x = np.empty(h.size, np.float32)
    lib().orc_f16_to_f32_n(_p(h), _p(x), h.size)
    return x


def tree_sum(x) -> np.float32:
    x = _c(x, np.float32)
    return np.float32(lib().orc_tree_sum(_p(x), x.size))


def dot(x, y) -> np.float32:
    x, y = _c(x, np.float32), _c(y, np.float32)
    return np.float32(lib().orc_dot(_p(x), _p(y), x.size))


# ----------------------------------------------------------------------------------------------
# one head of the plan and its packed segment
# ----------------------------------------------------------------------------------------------

DELTA_FIRST, DECAY_FIRST = 0, 1   # gate orders: A = Diag(a)(I - b k k^T) or (I - b k k^T) Diag(a)


class Head:
    """Static description of one head: per-row bits, pivot flags and row impact omega, and the
    gate order of its update (DELTA_FIRST, the literal A_t = Diag(a)(I - beta k k^T), or
    DECAY_FIRST, A_t = (I - beta k k^T) Diag(a))."""

    def __init__(self, bits, pivot, omega, dv=None, order=DELTA_FIRST):
        self.bits = _c(bits, np.int8)
        self.pivot = _c(pivot, np.uint8)
        self.omega = _c(omega, np.float32)
        self.dk = self.bits.size
        self.dv = self.dk if dv is None else dv
        self.order = int(order)

    @property
    def seg_bytes(self) -> int:
        return int(lib().orc_segment_bytes(self.dk, self.dv, _p(self.bits), _p(self.pivot)))

    def row_den(self) -> np.ndarray:
        den = np.empty(self.dk, np.float32)
        lib().orc_row_den(self.dk, _p(self.omega), _p(den))
        return den

    def encode(self, S, want_pre=False):
        S = _c(S, np.float32)
        seg = np.zeros(self.seg_bytes, np.uint8)
        pre = np.empty(self.dk * self.dv, np.float64) if want_pre else None
        fl = ctypes.c_uint32(0)
        lib().orc_encode(self.dk, self.dv, _p(self.bits), _p(self.pivot), _p(self.omega),
                         _p(S), _p(seg), _p(pre), ctypes.addressof(fl))
        return (seg, pre.reshape(self.dk, self.dv), fl.value) if want_pre else seg

    def unpack(self, seg):
        seg = _c(seg, np.uint8)
        S = np.empty((self.dk, self.dv), np.float32)
        r = np.empty(self.dk, np.uint16)
        c = np.empty(self.dv, np.uint16)
        z = np.empty((self.dk, self.dv), np.int8)
        rc = lib().orc_unpack(self.dk, self.dv, _p(self.bits), _p(self.pivot), _p(seg),
                              _p(S), _p(r), _p(c), _p(z))
        if rc != 0:
            raise ValueError("corrupt code (-2^(b-1)) in segment")
        return S, r, c, z

    def step(self, seg, q, k, v, a, beta, want_state=False):
        """In-place decode step of one tile; returns out (and S before requant, pre-round)."""
        q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
        a = _c(np.broadcast_to(np.asarray(a, np.float32), (self.dk,)), np.float32)
        out = np.empty(self.dv, np.float32)
        S = np.empty(self.dk * self.dv, np.float32) if want_state else None
        pre = np.empty(self.dk * self.dv, np.float64) if want_state else None
        fl = ctypes.c_uint32(0)
        rc = lib().orc_tile_step_o(self.dk, self.dv, _p(self.bits), _p(self.pivot),
                                 _p(self.omega), _p(seg), _p(q), _p(k), _p(v), _p(a),
                                 float(beta), _p(out), _p(S), _p(pre), ctypes.addressof(fl),
                                 self.order)
        if rc != 0:
            raise ValueError("corrupt code (-2^(b-1)) in segment")
        if want_state:
            return out, S.reshape(self.dk, self.dv), pre.reshape(self.dk, self.dv), fl.value
        return out


    def encode_dbg(self, S):
        """encode() with every intermediate the packed state does not show: returns
        (seg, dict(pre, z0, c0, flags)) -- pre the final pre-rounding values, z0 the first codes,
        c0 the first column factors."""
        S = _c(S, np.float32)
        seg = np.zeros(self.seg_bytes, np.uint8)
        pre = np.empty(self.dk * self.dv, np.float64)
        z0 = np.empty(self.dk * self.dv, np.int8)
        c0 = np.empty(self.dv, np.float32)
        fl = ctypes.c_uint32(0)
        lib().orc_encode_dbg(self.dk, self.dv, _p(self.bits), _p(self.pivot), _p(self.omega),
                             _p(S), _p(seg), _p(pre), _p(z0), _p(c0), ctypes.addressof(fl))
        return seg, dict(pre=pre.reshape(self.dk, self.dv), z0=z0.reshape(self.dk, self.dv),
                         c0=c0, flags=fl.value)

    def step_dbg(self, seg, q, k, v, a, beta):
        """step() in place on seg, returning dict(out, S (updated binary32 state), pre, z0, c0,
        flags)."""
        q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
        a = _c(np.broadcast_to(np.asarray(a, np.float32), (self.dk,)), np.float32)
        out = np.empty(self.dv, np.float32)
        S = np.empty(self.dk * self.dv, np.float32)
        pre = np.empty(self.dk * self.dv, np.float64)
        z0 = np.empty(self.dk * self.dv, np.int8)
        c0 = np.empty(self.dv, np.float32)
        fl = ctypes.c_uint32(0)
        rc = lib().orc_tile_step_dbg(self.dk, self.dv, _p(self.bits), _p(self.pivot),
                                     _p(self.omega), _p(seg), _p(q), _p(k), _p(v), _p(a),
                                     float(beta), _p(out), _p(S), _p(pre), _p(z0), _p(c0),
                                     ctypes.addressof(fl), self.order)
        if rc != 0:
            raise ValueError("corrupt code (-2^(b-1)) in segment")
        return dict(out=out, S=S.reshape(self.dk, self.dv), pre=pre.reshape(self.dk, self.dv),
                    z0=z0.reshape(self.dk, self.dv), c0=c0, flags=fl.value)


def fp32_step(S, q, k, v, a, beta, order=DELTA_FIRST):
    """FP32-state step on one tile in place; returns the readout."""
    dk, dv = S.shape
    q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
    a = _c(np.broadcast_to(np.asarray(a, np.float32), (dk,)), np.float32)
    out = np.empty(dv, np.float32)
    assert S.dtype == np.float32 and S.flags.c_contiguous
    lib().orc_fp32_step_o(dk, dv, _p(S), _p(q), _p(k), _p(v), _p(a), float(beta), _p(out),
                          int(order))
    return out


def fp32_run(S, q, k, v, a, beta, threads=8, want_out=False, order=DELTA_FIRST):
    """FP32-state steps on a batch of tiles.

    S: [N, dk, dv] float32 (updated in place).  q, k, v: [T, N, d]; a: [T, N, dk]; beta: [T, N].
    Returns out [T, N, dv] if want_out.  Tiles are split over threads; the result does not
    depend on the thread count (tiles are independent).
    """
    N, dk, dv = S.shape
    T = q.shape[0]
    q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
    a, beta = _c(a, np.float32), _c(beta, np.float32)
    assert S.dtype == np.float32 and S.flags.c_contiguous
    out = np.empty((T, N, dv), np.float32) if want_out else None
    nth = max(1, min(threads, N))
    bounds = np.linspace(0, N, nth + 1).astype(int)
    # each thread takes a contiguous tile range; its beta slice is gathered into a private array
    def work(t0, t1):
        n = t1 - t0
        if n == 0:
            return
        b = np.ascontiguousarray(beta[:, t0:t1])
        lib().orc_fp32_run_o(dk, dv, n, T, S[t0:].ctypes.data, q[:, t0:].ctypes.data,
                           k[:, t0:].ctypes.data, v[:, t0:].ctypes.data, N * dv,
                           a[:, t0:].ctypes.data, N * dk, _p(b),
                           None if out is None else out[:, t0:].ctypes.data, int(order))
    with ThreadPoolExecutor(nth) as ex:
        list(ex.map(lambda ab: work(*ab), zip(bounds[:-1], bounds[1:])))
    return out


# ----------------------------------------------------------------------------------------------
# offline inputs (binary64): Method 1 and Method 2
# ----------------------------------------------------------------------------------------------

def lifetime_weight(l_u, H: int) -> np.ndarray:
    """L_u = sum_{j=0}^{H-1} exp(2 j l_u), the error-lifetime weight over the next H steps
    (Method 1), summed term by term as printed."""
    l_u = np.asarray(l_u, np.float64)
    j = np.arange(H, dtype=np.float64)
    return np.array([np.sum(np.exp(2.0 * j * lu)) for lu in l_u.ravel()]).reshape(l_u.shape)


def row_impact(q, k, a, beta, order=DELTA_FIRST) -> np.ndarray:
    """omega_i = E[g_i^2] with g = A^T q (Method 2): for A = Diag(a)(I - b k k^T),
    g = a*q - beta k (k . (a*q)); for A = (I - b k k^T) Diag(a), g = a * (q - beta k (k . q)).
    q, k, a: [n, dk] samples of one head; beta: [n].  Mean over samples."""
    q, k, a = (np.asarray(x, np.float64) for x in (q, k, a))
    beta = np.asarray(beta, np.float64)
    if order == DECAY_FIRST:
        g = a * (q - (beta * np.sum(k * q, axis=-1))[:, None] * k)
    else:
        aq = a * q
        g = aq - (beta * np.sum(k * aq, axis=-1))[:, None] * k
    return np.mean(g * g, axis=0)


def select_pivots(risk, n_pivots: int) -> np.ndarray:
    """Indices of the n_pivots units of largest risk = L_u d_u(b_max); ties to the lower index
    (the pages keep a few FP16 pivots for the hardest units, Method 1)."""
    risk = np.asarray(risk, np.float64)
    order = sorted(range(risk.size), key=lambda u: (-risk[u], u))
    return np.array(sorted(order[:n_pivots]), dtype=np.int64)


def mcdp_allocate(cost, choices, capacity_bits: int):
    """Multiple-choice DP over equal-size units (Method 1, GDN unit = head).

    cost[u][c] = L_u d_u(choices[c]); choices ascending even widths; the budget is
    sum_u b_u <= capacity_bits.  Minimises sum_u cost[u][b_u].  A state holds the exact bit
    total reached (in steps of two bits); among equal costs a choice with fewer bits wins
    (choices are tried in ascending order and replace the incumbent only when strictly
    cheaper), and the final total is the cheapest, then smallest, feasible one.
    Returns (bits per unit, objective)."""
    cost = np.asarray(cost, np.float64)
    choices = [int(b) for b in choices]
    N = cost.shape[0]
    cap = capacity_bits // 2
    w = [b // 2 for b in choices]
    INF = float("inf")
    dp = [0.0] + [INF] * cap
    pick = np.full((N, cap + 1), -1, np.int16)
    for u in range(N):
        nd = [INF] * (cap + 1)
        for c in range(cap + 1):
            for ci, wc in enumerate(w):
                if c - wc < 0 or dp[c - wc] == INF:
                    continue
                val = dp[c - wc] + float(cost[u, ci])
                if val < nd[c]:
                    nd[c] = val
                    pick[u, c] = ci
        dp = nd
    best_c, best = -1, INF
    for c in range(cap + 1):
        if dp[c] < best:
            best, best_c = dp[c], c
    if best_c < 0:
        raise ValueError("budget too small for the smallest width")
    out = np.empty(N, np.int64)
    c = best_c
    for u in range(N - 1, -1, -1):
        ci = int(pick[u, c])
        out[u] = choices[ci]
        c -= w[ci]
    return out, best


def lagrangian_allocate(L, d, n, choices, budget_bits: float, iters: int = 100):
    """Lagrangian allocation with discrete budget repair (Method 1, KDA unit = key row).

    Minimises sum_u L_u d_u(b_u) subject to sum_u n_u b_u <= budget_bits.
    b_u(lam) = argmin_b L_u d_u(b) + lam n_u b (ties to the smaller width).  hi doubles from 1
    until feasible, then bisection (iters halvings) keeps the feasible end.  Repair: repeatedly
    take the single-step upgrade (to the next allowed width) with the largest
    (L_u (d_u(b) - d_u(b'))) / (n_u (b' - b)) that still fits, ties to the lower unit, until none
    fits.  Returns (bits per unit, objective)."""
    L = np.asarray(L, np.float64)
    d = np.asarray(d, np.float64)
    n = np.asarray(n, np.float64)
    choices = [int(b) for b in choices]
    N = L.size

    def assign(lam):
        b = np.empty(N, np.int64)
        for u in range(N):
            best, bi = None, 0
            for ci, bc in enumerate(choices):
                val = L[u] * d[u, ci] + lam * n[u] * bc
                if best is None or val < best:
                    best, bi = val, ci
            b[u] = bi
        return b

    def total(bi):
        return float(sum(n[u] * choices[bi[u]] for u in range(N)))

    hi = 1.0
    while total(assign(hi)) > budget_bits:
        hi *= 2.0
        if hi > 1e300:
            raise ValueError("budget too small for the smallest width")
    lo = 0.0
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if total(assign(mid)) <= budget_bits:
            hi = mid
        else:
            lo = mid
    bi = assign(hi)
    used = total(bi)
    while True:
        best, bu = None, -1
        for u in range(N):
            ci = bi[u]
            if ci + 1 >= len(choices):
                continue
            extra = n[u] * (choices[ci + 1] - choices[ci])
            if used + extra > budget_bits:
                continue
            gain = (L[u] * (d[u, ci] - d[u, ci + 1])) / extra
            if best is None or gain > best:
                best, bu = gain, u
        if bu < 0 or best <= 0.0:
            break
        used += n[bu] * (choices[bi[bu] + 1] - choices[bi[bu]])
        bi[bu] += 1
    b = np.array([choices[c] for c in bi], np.int64)
    obj = float(sum(L[u] * d[u, bi[u]] for u in range(N)))
    return b, obj


def objective(L, d, choices, b) -> float:
    idx = {int(c): i for i, c in enumerate(choices)}
    L = np.asarray(L, np.float64)
    d = np.asarray(d, np.float64)
    return float(sum(L[u] * d[u, idx[int(b[u])]] for u in range(len(b))))
