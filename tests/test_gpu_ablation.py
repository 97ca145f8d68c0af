"""Baseline and ablation plans through the decode kernels, and their drift against an FP32
state (quantized_delta_rule_amd.ablation).  The FP32 reference of that report is itself pinned
to the oracle's FP32-state run."""
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


@pytest.mark.parametrize("wid", [2, 4])
def test_fp32_reference_matches_oracle(gpu, wid):
    """The FP32 recurrence of the product side (plain torch: initial and calibration states, the
    drift reference) against the oracle's FP32-state run on
    the same inputs: both sum in binary32 in different orders, so they agree to ~1e-6."""
    torch = gpu
    from quantized_delta_rule_amd import reference
    w = dataclasses.replace(synth.WORKLOADS[wid], B=2, H=3, warmup=12)
    dev = torch.device("cuda:0")
    S_t = reference.warm_state(w, 0, dev)
    S_o = P.warm_state(w, 0)
    assert P.rel_l2(S_t.cpu().numpy(), S_o) < 1e-5
    for s in range(6):
        xh = synth.step_inputs(w, 0, s, "decode")
        x = reference.device_inputs(xh, w, dev)
        o_t = reference.fp32_step(S_t, x["q"], x["k"], x["v"], x["a"], x["beta"]).cpu().numpy()
        a_rows = synth.alpha_rows(w, xh["alpha"])
        for t in range(w.B * w.H):
            b, h = divmod(t, w.H)
            o = oracle.fp32_step(S_o[t], xh["q"][b, h], xh["k"][b, h], xh["v"][b, h],
                                 a_rows[b, h], xh["beta"][b, h])
            assert P.rel_l2(o_t[t], o) < 1e-5
    assert P.rel_l2(S_t.cpu().numpy(), S_o) < 1e-5


def test_variant_drift(gpu):
    """Every variant runs through the kernels with no status flag; uniform plans drift less as
    their width grows; all drift stays below the state's own scale (requantizing every step
    accumulates error until the gate's decay balances it: about 0.3 at 4 bits)."""
    from quantized_delta_rule_amd import ablation
    w = dataclasses.replace(synth.WORKLOADS[2], B=6, H=8)
    res = ablation.drift(w, 24, log=P.log)
    for name, r in res.items():
        P.log(f"[drift] {name}: {r}")
        for k, v in r.items():
            assert np.isfinite(v), (name, k)
        assert r["readout_rel_l2_max"] < 1.0, name
    s = [res[f"uniform-{b}"]["state_rel_l2_last"] for b in (4, 6, 8)]
    assert s[0] > s[1] > s[2], s
    # the budgeted plans store about the nominal width
    assert abs(res["stepquant"]["bits_per_value"] - res["temporal"]["bits_per_value"]) < 1e-9
