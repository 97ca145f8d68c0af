"""Calibration estimators on the device: row impact (stepq_row_impact_gpu) against the oracle's
binary64 row impact, and the measured distortion table (library encode + decode of calibration
states) against the same measurement made with the oracle's quantizer."""
import dataclasses

import numpy as np
import pytest

import oracle
import paritylib as P
from quantized_delta_rule_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from quantized_delta_rule_amd import stepq
    stepq.lib()
    return torch


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("kind,d", [("gdn", 128), ("kda", 64), ("kda", 128), ("gdn", 64)])
def test_row_impact_gpu_matches_oracle(gpu, kind, d, order):
    from quantized_delta_rule_amd import planning
    base = synth.WORKLOADS[2 if kind == "gdn" else 4]
    w = dataclasses.replace(base, B=5, H=3, d=d, calib_steps=0, warmup=4, order=order)
    om_gpu = planning.omega_gpu(w, 0)
    om_orc = P.omega_from_steps(w, 0, "warmup", w.warmup)
    om_host = planning.omega(w, 0)
    # binary64 sums in different orders, rounded to binary32: equal up to the last bit or two
    np.testing.assert_allclose(om_gpu, om_orc, rtol=3e-7, atol=0)
    np.testing.assert_allclose(om_host, om_orc, rtol=3e-7, atol=0)


def test_row_impact_gpu_accumulates_and_handles_empty_batch(gpu):
    torch = gpu
    from quantized_delta_rule_amd import stepq
    dev = torch.device("cuda:0")
    w = dataclasses.replace(synth.WORKLOADS[2], B=4, H=2, d=64)
    acc = torch.zeros(w.H * w.d, dtype=torch.float64, device=dev)
    x = {k: torch.from_numpy(v).to(dev) for k, v in synth.step_inputs(w, 0, 0).items()}
    stepq.row_impact_gpu(stepq.GDN, x["q"], x["k"], x["alpha"], x["beta"], acc)
    once = acc.clone()
    stepq.row_impact_gpu(stepq.GDN, x["q"], x["k"], x["alpha"], x["beta"], acc)
    torch.testing.assert_close(acc, 2 * once, rtol=1e-15, atol=0)
    stepq.row_impact_gpu(stepq.GDN, x["q"][:0], x["k"][:0], x["alpha"][:0], x["beta"][:0], acc)
    torch.testing.assert_close(acc, 2 * once, rtol=0, atol=0)


@pytest.mark.parametrize("kind", ["kda", "gdn"])
def test_measured_distortion_matches_oracle_measurement(gpu, kind):
    """Same recipe on both sides: calibration states from zero, uniform-width plans without
    pivots, squared error summed per row.  The GPU side builds its states with the torch FP32
    recurrence and quantizes with the kernels; the oracle side uses its own FP32 run and
    quantizer.  The states differ in the last bits (summation order), so the tables agree to a
    relative 1e-3 rather than exactly."""
    from quantized_delta_rule_amd import planning
    base = synth.WORKLOADS[4 if kind == "kda" else 6]
    w = dataclasses.replace(base, H=2, calib_steps=8, layers=1)
    om = P.omega_from_steps(w, 0, "calib", w.calib_steps)
    du_gpu = planning.measured_distortion_gpu(w, 0, om, n_req=3, samples=(6, 12))
    du_orc = P.measured_distortion(w, om[None], n_req=3, samples=(6, 12))[0]
    P.log(f"[calib] {kind} d_u gpu {du_gpu[0, :2]} oracle {du_orc[0, :2]}")
    np.testing.assert_allclose(du_gpu, du_orc, rtol=1e-3, atol=0)
    # more bits, less distortion, for every row
    assert np.all(np.diff(du_gpu, axis=-1) < 0)


def test_calibrated_plan_respects_budget(gpu):
    """The calibrated GDN allocation (measured table, lifetime weights) keeps the nominal
    budget over non-pivot heads and picks the configured number of pivots."""
    from quantized_delta_rule_amd import planning
    w = dataclasses.replace(synth.WORKLOADS[6], B=4, H=8)
    bits, piv, om = planning.plan_arrays(w)
    head_bits = bits[0, :, 0]
    head_piv = piv[0, :, 0].astype(bool)
    assert head_piv.sum() == w.n_pivots
    assert head_bits[~head_piv].sum() <= w.nominal * (~head_piv).sum()
    assert set(head_bits[~head_piv]) <= set(w.choices)
