"""Product-side offline planning for a synthetic workload, through libstepq's host planners.

Page: "STEPQuant" paper digest (vibe-research silicon-writer readme), Method 1 (lifetime weight
L_u = sum_{j<H} exp(2 j l_u), allocation minimising sum_u L_u d_u(b_u) under an average-bit
budget -- multiple-choice DP for GDN heads, Lagrangian with budget repair for KDA rows -- and a
few FP16 pivot units for the hardest units) and Method 2 (row impact omega_i = E[g_i^2] with
g = A^T q).
"""
from __future__ import annotations

import numpy as np

from . import reference, stepq, synth


def _calib_phase(w: synth.Workload):
    """Input stream and step count the row impact is estimated on."""
    return ("calib", w.calib_steps) if w.calib_steps else ("warmup", w.warmup)


def omega(w: synth.Workload, layer: int, phase: str | None = None, steps: int | None = None):
    """Row impact [H, d] accumulated by the library's host planner over the given input steps
    (default: the workload's calibration stream)."""
    dphase, dsteps = _calib_phase(w)
    phase = dphase if phase is None else phase
    steps = dsteps if steps is None else steps
    acc = np.zeros((w.H, w.d))
    n = 0
    for x in synth.step_inputs_many(w, layer, range(steps), phase):
        a = synth.alpha_rows(w, x["alpha"])
        for h in range(w.H):
            stepq.row_impact_accumulate(x["q"][:, h], x["k"][:, h], a[:, h], x["beta"][:, h],
                                        acc[h], order=w.order)
        n += w.B
    return (acc / n).astype(np.float32)


def omega_gpu(w: synth.Workload, layer: int, phase: str | None = None,
              steps: int | None = None, device: int = 0):
    """The same row impact [H, d], accumulated on the device (stepq_row_impact_gpu)."""
    import torch
    dphase, dsteps = _calib_phase(w)
    phase = dphase if phase is None else phase
    steps = dsteps if steps is None else steps
    dev = torch.device(f"cuda:{device}")
    acc = torch.zeros(w.H * w.d, dtype=torch.float64, device=dev)
    kind = stepq.GDN if w.kind == "gdn" else stepq.KDA
    for s in range(steps):
        x = {k: torch.from_numpy(v).to(dev) for k, v in synth.step_inputs(w, layer, s, phase).items()}
        stepq.row_impact_gpu(kind, x["q"], x["k"], x["alpha"], x["beta"], acc, order=w.order)
    return (acc / (w.B * steps)).to(torch.float32).cpu().numpy().reshape(w.H, w.d)


def measured_distortion_gpu(w: synth.Workload, layer: int, omega_l, n_req: int = 8,
                            samples=(32, 64), device: int = 0):
    """d(b) per key row [H, d, len(choices)]: the squared reconstruction error summed over the
    row, of the uniform-width-b plan (no pivots) encoded and decoded by the library's kernels,
    averaged over calibration states (n_req requests run from zero on the calibration stream,
    states at the sample steps).  Method 1: the allocation's reconstruction distortion d_u(b),
    measured rather than modelled."""
    import torch
    dev = torch.device(f"cuda:{device}")
    kind = stepq.GDN if w.kind == "gdn" else stepq.KDA
    H, d = w.H, w.d
    n_req = min(n_req, w.B)
    states = reference.calib_states(w, layer, dev, n_req, samples)
    du = torch.zeros((H, d, len(w.choices)), dtype=torch.float64, device=dev)
    for ci, b in enumerate(w.choices):
        plan = stepq.Plan(kind, np.full((H, d), b, np.int8), np.zeros((H, d), np.uint8), omega_l,
                          device=device, order=w.order)
        pool = plan.alloc_pool(n_req)
        for S in states:
            plan.encode(S, pool, n_req)
            S_hat = plan.unpack(pool, n_req)[0].reshape(n_req * H, d, d)
            err = ((S.double() - S_hat.double()) ** 2).sum(-1)        # [n_req*H, d]
            du[:, :, ci] += err.reshape(n_req, H, d).sum(0)
        if plan.status() != 0:
            raise RuntimeError(f"width {b}: status flags raised while measuring d_u")
        plan.close()
    return (du / (len(states) * n_req)).cpu().numpy()


def calibrate(w: synth.Workload, device: int = 0):
    """Row impact [layers, H, d] and the measured distortion table [units, choices] (units:
    layers*H heads for GDN, layers*H*d key rows for KDA), both from the library's kernels."""
    om = np.stack([omega_gpu(w, l, device=device) for l in range(w.layers)])
    du = np.stack([measured_distortion_gpu(w, l, om[l], device=device) for l in range(w.layers)])
    if w.kind == "gdn":
        du = du.sum(axis=2)                       # a head's distortion: sum over its rows
    return om, du.reshape(-1, len(w.choices))


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
    """(bits, pivot, omega), each [layers, H, d], for the workload.  A workload with a measured
    distortion table is calibrated on the device first (calibrate)."""
    Lr, H, d = w.layers, w.H, w.d
    if w.du == "measured" and distortion is None and w.alloc != "fixed":
        om_c, distortion = calibrate(w)
        omegas = om_c if omegas is None else omegas
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


def code_bytes(w: synth.Workload, plan: "stepq.Plan") -> int:
    """Packed-state bytes of one layer read once (codes, binary16 factors and pivots): what the
    split mode's side-stream writeback reads a second time."""
    d = w.d
    total = 0
    for h in range(plan.H):
        b = plan.bits[h]
        p = plan.pivot[h].astype(bool)
        total += d * int(b[~p].astype(np.int64).sum()) // 8 + 2 * d * int(p.sum())
        if (~p).any():
            total += 2 * (d + d)
    return w.B * total


# Algorithmic ALU operations per state entry of one decode step, counted from the binary32
# evaluation order the kernels follow (each multiply, add, fused multiply-add, maximum, rounding,
# clamp, conversion and code extraction/insertion counts one; reductions over 128 rows cost
# 128 leaves + 31 tree additions per column):
#   dequantize 3 (extract, convert, x c_j) | k^T S 1.242 | update 1 (T = fma(K_i, e_j, X))
#   q^T S 1.242 | row magnitude 0.992 | y = T rho_i 1 | column maximum 1 (KDA: 2, the per-row
#   1/qmax) | first quantization 1 | least-squares sums 3.484 | final quantization, clamp, pack 3
# KDA adds one per entry for its per-row error e_ij = v_j - a_i u_j.  FP16 pivot rows: convert 1,
# k^T S, update, q^T S, row magnitude, convert back 1.  Per-row and per-column work (factors and
# their reciprocals) adds about 0.1 per entry.
OPS_QUANT_GDN = 3 + 1.242 + 1 + 1.242 + 0.992 + 1 + 1 + 1 + 3.484 + 3 + 0.1
OPS_QUANT_KDA = OPS_QUANT_GDN + 2
OPS_PIVOT = 1 + 1.242 + 1 + 1.242 + 0.992 + 1 + 0.1


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
