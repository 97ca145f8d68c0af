"""Product-side offline planning for a synthetic workload, through libstepq's host planners.

Page: "STEPQuant" paper digest (vibe-research silicon-writer readme), Method 1 (lifetime weight
L_u = sum_{j<H} exp(2 j l_u), allocation minimising sum_u L_u d_u(b_u) under an average-bit
budget -- multiple-choice DP for GDN heads, Lagrangian with budget repair for KDA rows -- and a
few FP16 pivot units for the hardest units) and Method 2 (row impact omega_i = E[g_i^2] with
g = A^T q).
"""
from __future__ import annotations

import numpy as np

from . import stepq, synth


def omega(w: synth.Workload, layer: int, phase: str = "warmup", steps: int | None = None):
    """Row impact [H, d] accumulated by the library over the given input steps."""
    steps = w.warmup if steps is None else steps
    acc = np.zeros((w.H, w.d))
    n = 0
    for s in range(steps):
        x = synth.step_inputs(w, layer, s, phase)
        a = synth.alpha_rows(w, x["alpha"])
        for h in range(w.H):
            stepq.row_impact_accumulate(x["q"][:, h], x["k"][:, h], a[:, h], x["beta"][:, h],
                                        acc[h])
        n += w.B
    return (acc / n).astype(np.float32)


def allocate(w: synth.Workload, distortion=None):
    """Per-unit widths and pivot flags for the workload's units (GDN heads over all layers, or
    KDA key rows).  distortion: [units, choices] table, or None for the synthetic one."""
    l_u, s_u = synth.plan_tables(w)
    L = stepq.lifetime_weights(l_u, w.horizon)
    choices = list(w.choices)
    du = synth.synthetic_distortion(s_u, choices) if distortion is None else distortion
    piv_idx = stepq.select_pivots(L * du[:, -1], w.n_pivots)
    keep = np.setdiff1d(np.arange(L.size), piv_idx)
    if w.alloc == "mcdp":
        b_keep, _ = stepq.alloc_mcdp(L[keep, None] * du[keep], choices, w.nominal * keep.size)
    else:
        n = np.full(keep.size, float(w.d))
        b_keep, _ = stepq.alloc_lagrangian(L[keep], du[keep], n, choices,
                                           w.nominal * float(n.sum()))
    bits = np.full(L.size, max(choices), np.int64)
    bits[keep] = b_keep
    piv = np.zeros(L.size, np.uint8)
    piv[piv_idx] = 1
    return bits, piv


def plan_arrays(w: synth.Workload, omegas=None, distortion=None):
    """(bits, pivot, omega), each [layers, H, d], for the workload."""
    Lr, H, d = w.layers, w.H, w.d
    if omegas is None:
        omegas = np.stack([omega(w, l) for l in range(Lr)])
    bits = np.zeros((Lr, H, d), np.int8)
    piv = np.zeros((Lr, H, d), np.uint8)
    if w.alloc == "fixed":
        for h, b in enumerate(w.fixed_bits):
            bits[:, h] = b if b else max(w.choices)
            piv[:, h] = 0 if b else 1
        return bits, piv, omegas
    ub, up = allocate(w, distortion)
    if w.kind == "gdn":
        bits[:] = ub.reshape(Lr, H)[:, :, None]
        piv[:] = up.reshape(Lr, H)[:, :, None]
    else:
        bits[:] = ub.reshape(Lr, H, d)
        piv[:] = up.reshape(Lr, H, d)
    return bits, piv, omegas


def algorithmic_bytes(w: synth.Workload, plan: "stepq.Plan") -> int:
    """Bytes one decode step of one layer must move: every head's packed state read and written
    once (codes, binary16 factors, binary16 pivots; segment padding excluded), plus q, k, v,
    alpha, beta in and out out."""
    d = w.d
    per_req = 0
    for h in range(plan.H):
        b = plan.bits[h]
        p = plan.pivot[h].astype(bool)
        payload = d * int(b[~p].astype(np.int64).sum()) // 8 + 2 * d * int(p.sum())
        if (~p).any():
            payload += 2 * (d + d)
        per_req += 2 * payload
    a_bytes = 4 * (d if w.kind == "kda" else 1)
    io = plan.H * (3 * 4 * d + a_bytes + 4 + 4 * d)
    return w.B * (per_req + io)


# Algorithmic ALU operations per state entry of one decode step, counted from the evaluation
# order of the method (each binary32 multiply, add, fused multiply-add, maximum, rounding, clamp,
# conversion and code extraction/insertion counts one; reductions over 128 rows cost
# 128 leaves + 31 tree additions per column):
#   dequantize 3 (extract, convert, x c_j) | k^T S 1.242 | update 2 | q^T S 1.242
#   row magnitude 0.992 | y = S / r 1 | column maximum 1 (KDA: 2, the per-row 1/qmax)
#   first quantization 1 | least-squares sums 3.484 | final quantization, clamp, pack 3
# KDA adds one per entry for its per-row e = v - a_i u.  FP16 pivot rows: convert 1, k^T S,
# update, q^T S, row magnitude, convert back 1.  Per-row and per-column work (factors and their
# reciprocals) adds about 0.1 per entry.
OPS_QUANT_GDN = 3 + 1.242 + 2 + 1.242 + 0.992 + 1 + 1 + 1 + 3.484 + 3 + 0.1
OPS_QUANT_KDA = OPS_QUANT_GDN + 2
OPS_PIVOT = 1 + 1.242 + 2 + 1.242 + 0.992 + 1 + 0.1


def algorithmic_ops(w: synth.Workload, plan: "stepq.Plan") -> float:
    """ALU operations one decode step of one layer performs (see the table above)."""
    d = w.d
    per_req = 0.0
    for h in range(plan.H):
        p = plan.pivot[h].astype(bool)
        nq, npv = int((~p).sum()), int(p.sum())
        per_req += d * (nq * (OPS_QUANT_KDA if w.kind == "kda" else OPS_QUANT_GDN)
                        + npv * OPS_PIVOT)
    return w.B * per_req
