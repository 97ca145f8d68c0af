"""Drift of the packed-state decode path against an FP32 state, for STEPQuant and the baseline and
ablation plans, all through the same kernels.

Page: "STEPQuant" paper digest (vibe-research silicon-writer readme).  Its ablation compares the
full method with variants that drop one axis: uniform widths without the impact weighting (a
plain uniform INT-b state), the lifetime-aware allocation alone (temporal only) and the
impact-weighted dual-axis fitting alone (spatial only); the digest reports them against an FP32
state.  Here every variant is only a different plan -- widths, pivots and row impact -- for the
one decode kernel:

  uniform-b   every unit at width b, no pivots, omega = 1 (the fit then weights rows evenly)
  spatial     every unit at the nominal width, no pivots, measured omega
  temporal    lifetime-weighted allocation with FP16 pivots (Method 1), omega = 1
  stepquant   lifetime-weighted allocation, pivots and measured omega (Methods 1-3)

The reference is the FP32-state recurrence S_t = A_t S_{t-1} + beta k v^T, o_t = S_t^T q_t in
plain PyTorch fp32 on the same seeded inputs and initial state.  Reported per variant: stored
bits per value, the readout's relative L2 error per step (mean, max and last over the run) and
the state's relative L2 error after the last step.

    python -m quantized_delta_rule_amd.ablation --workload 2 --steps 64
"""
from __future__ import annotations

import argparse
import json
import sys

import numpy as np

from . import planning, reference, stepq, synth


def variant_plans(w: synth.Workload, layer: int = 0):
    """{name: (bits, pivot, omega)} for one layer, each [H, d]."""
    H, d = w.H, w.d
    om = planning.omega(w, layer)
    ones = np.ones((H, d), np.float32)
    nopiv = np.zeros((H, d), np.uint8)
    plans = {}
    for b in w.choices:
        plans[f"uniform-{b}"] = (np.full((H, d), b, np.int8), nopiv, ones)
    plans["spatial"] = (np.full((H, d), w.nominal, np.int8), nopiv, om)
    bits, piv, _ = planning.plan_arrays(w, omegas=np.stack([om] * w.layers))
    plans["temporal"] = (bits[layer], piv[layer], ones)
    plans["stepquant"] = (bits[layer], piv[layer], om)
    return plans


def _rel(a, b):
    return float((a - b).double().norm() / max(float(b.double().norm()), 1e-300))


def drift(w: synth.Workload, steps: int, layer: int = 0, variants=None, device=0, log=None):
    """Runs every variant and the FP32 reference in lockstep on the same inputs.  Returns
    {name: {...metrics...}}."""
    import torch
    dev = torch.device(f"cuda:{device}")
    kind = stepq.GDN if w.kind == "gdn" else stepq.KDA
    plans = variant_plans(w, layer)
    if variants is not None:
        plans = {k: v for k, v in plans.items() if k in variants}
    S_ref = reference.warm_state(w, layer, dev)
    runs = {}
    for name, (bits, piv, om) in plans.items():
        p = stepq.Plan(kind, bits, piv, om, device=device)
        pool = p.alloc_pool(w.B)
        p.encode(S_ref, pool, w.B)
        runs[name] = (p, pool, [])
    B, H, d = w.B, w.H, w.d
    out = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    for s in range(steps):
        x = reference.device_inputs(synth.step_inputs(w, layer, s, "decode"), w, dev)
        o_ref = reference.fp32_step(S_ref, x["q"], x["k"], x["v"], x["a"], x["beta"]).reshape(B, H, d)
        for name, (p, pool, errs) in runs.items():
            p.step(pool, B, x["q"], x["k"], x["v"], x["alpha"], x["beta"], out)
            errs.append(_rel(out, o_ref))
        if log and (s + 1) % max(1, steps // 4) == 0:
            log(f"[drift] {w.name}: step {s + 1}/{steps}")
    res = {}
    for name, (p, pool, errs) in runs.items():
        S_hat = p.unpack(pool, B)[0].reshape(B * H, d, d)
        if p.status() != 0:
            raise RuntimeError(f"variant {name}: status flags raised")
        e = np.asarray(errs)
        res[name] = {"bits_per_value": round(p.bits_per_value, 4),
                     "readout_rel_l2_mean": float(e.mean()), "readout_rel_l2_max": float(e.max()),
                     "readout_rel_l2_last": float(e[-1]), "state_rel_l2_last": _rel(S_hat, S_ref)}
        p.close()
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--layer", type=int, default=0)
    args = ap.parse_args(argv)
    w = synth.WORKLOADS[args.workload]
    res = drift(w, args.steps, args.layer,
                log=lambda m: print(m, file=sys.stderr, flush=True))
    for name, r in res.items():
        print(json.dumps({"workload": w.name, "steps": args.steps, "variant": name, **r}),
              flush=True)


if __name__ == "__main__":
    main()
