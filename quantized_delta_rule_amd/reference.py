"""FP32-state Delta-rule recurrence in plain PyTorch: initial states for the decode pool,
calibration states, and the reference of the drift report.  This is not the decode path (that
runs only in libstepq's kernels); it supplies the unquantized states the method starts from and
is compared against.

Page: "STEPQuant" paper digest (vibe-research silicon-writer readme), Background:
S_t = A_t S_{t-1} + beta_t k_t v_t^T with A_t = Diag(a)(I - beta_t k_t k_t^T), o_t = S_t^T q_t
(a = alpha broadcast over the rows for GDN, per row for KDA).
"""
from __future__ import annotations

import numpy as np

from . import synth


def fp32_step(S, q, k, v, a, beta):
    """One step on tiles S [N, d_k, d_v] in place; returns o [N, d_v].  q, k, a [N, d_k],
    v [N, d_v], beta [N]."""
    u = (S * k[:, :, None]).sum(1)                          # S^T k
    e = v[:, None, :] - a[:, :, None] * u[:, None, :]       # v - a_i u
    S.mul_(a[:, :, None]).add_((beta[:, None] * k)[:, :, None] * e)
    return (S * q[:, :, None]).sum(1)


def device_inputs(x, w: synth.Workload, dev, n_req=None):
    """Step inputs on the device, flattened over (request, head): q, k, v, a [N, d], beta [N]
    and alpha as the decode call takes it; optionally only the first n_req requests."""
    import torch
    d = w.d
    sl = slice(None) if n_req is None else slice(0, n_req)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return {"q": t(x["q"][sl].reshape(-1, d)), "k": t(x["k"][sl].reshape(-1, d)),
            "v": t(x["v"][sl].reshape(-1, d)),
            "a": t(synth.alpha_rows(w, x["alpha"][sl]).reshape(-1, d)),
            "beta": t(x["beta"][sl].reshape(-1)), "alpha": t(x["alpha"][sl])}


def warm_state(w: synth.Workload, layer: int, dev, xs=None):
    """Initial states [B*H, d, d]: w.warmup steps from zero on the warm-up stream (xs: those
    steps' inputs if already drawn)."""
    import torch
    S = torch.zeros((w.B * w.H, w.d, w.d), dtype=torch.float32, device=dev)
    if xs is None:
        xs = synth.step_inputs_many(w, layer, range(w.warmup), "warmup")
    for x_ in xs:
        x = device_inputs(x_, w, dev)
        fp32_step(S, x["q"], x["k"], x["v"], x["a"], x["beta"])
    return S


def calib_states(w: synth.Workload, layer: int, dev, n_req=8, samples=(32, 64)):
    """Calibration states: n_req requests run from zero on the calibration stream; a copy of
    the states [n_req*H, d, d] at each sample step."""
    import torch
    S = torch.zeros((n_req * w.H, w.d, w.d), dtype=torch.float32, device=dev)
    out, s = [], 0
    for smp in samples:
        while s < smp:
            x = device_inputs(synth.step_inputs(w, layer, s, "calib"), w, dev, n_req)
            fp32_step(S, x["q"], x["k"], x["v"], x["a"], x["beta"])
            s += 1
        out.append(S.clone())
    return out
