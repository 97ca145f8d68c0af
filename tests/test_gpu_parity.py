"""GPU <-> oracle parity through the C ABI (needs an MI355X and the built library)."""
import dataclasses

import numpy as np
import pytest

import paritylib as P
from quantized_delta_rule_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from quantized_delta_rule_amd import stepq
    stepq.lib()
    return torch


def _small(wid, kind="gdn", d=128, B=3, H=4, steps=6, **kw):
    return synth.Workload(wid, f"case{wid}", kind, B=B, layers=1, H=H, d=d, steps=steps,
                          warmup=8, choices=(4, 6, 8), nominal=6, n_pivots=0,
                          alloc="fixed", **kw)


def test_workload1_every_tile_every_step(torch_gpu):
    w = synth.WORKLOADS[1]
    P.log(f"[parity] workload 1 {w.name}: B={w.B} H={w.H} d={w.d} steps={w.steps}")
    bits, piv, om = P.oracle_plan(w)
    tr, plan, _ = P.run_layer(w, 0, bits[0], piv[0], om[0], w.steps)
    P.log(f"[parity] workload 1 ok: boundary={tr.boundary} worst readout={tr.worst_readout:.2e}")
    assert plan.status() == 0


@pytest.mark.parametrize("b", [2, 4, 6, 8])
@pytest.mark.parametrize("d", [64, 128])
def test_gdn_each_width(torch_gpu, b, d):
    w = _small(200 + b + d, d=d, H=2, fixed_bits=(b, 0))
    P.log(f"[parity] GDN width {b} d={d}")
    bits, piv, om = P.oracle_plan(w)
    tr, plan, _ = P.run_layer(w, 0, bits[0], piv[0], om[0], w.steps)
    assert plan.status() == 0


@pytest.mark.parametrize("d", [64, 128])
def test_kda_mixed_rows_and_pivots(torch_gpu, d):
    w = _small(300 + d, kind="kda", d=d, H=3)
    P.log(f"[parity] KDA mixed d={d}")
    g = np.random.default_rng(d)
    bits = g.choice([2, 4, 6, 8], size=(w.H, d)).astype(np.int8)
    piv = np.zeros((w.H, d), np.uint8)
    piv[0, [0, 5, d - 1]] = 1
    piv[1, g.choice(d, 9, replace=False)] = 1
    om = P.omega_from_steps(w, 0, "warmup", w.warmup)
    tr, plan, _ = P.run_layer(w, 0, bits, piv, om, w.steps)
    assert plan.status() == 0


def test_dead_rows_columns_and_identity_step(torch_gpu):
    w = _small(401, d=128, B=2, H=2, fixed_bits=(6, 4))
    bits, piv, om = P.oracle_plan(w)
    S0 = P.warm_state(w, 0)
    S0[0, 3, :] = 0.0      # dead row
    S0[1, :, 7] = 0.0      # dead column
    S0[2] = 0.0            # all-zero tile
    d = w.d

    def inputs(s):  # alpha = 1, beta = 0: the decoded state passes through unchanged
        x = synth.step_inputs(w, 0, s)
        x["alpha"][:] = 1.0
        x["beta"][:] = 0.0
        return x
    P.log("[parity] dead rows/columns, identity steps")
    tr, plan, _ = P.run_layer(w, 0, bits[0], piv[0], om[0], 3, S0=S0, inputs=inputs)
    assert plan.status() == 0


def test_empty_batch_is_a_no_op(torch_gpu):
    import torch
    from quantized_delta_rule_amd import stepq
    w = _small(402, B=1, H=2, fixed_bits=(6, 0))
    bits, piv, om = P.oracle_plan(w)
    plan = stepq.Plan(stepq.GDN, bits[0], piv[0], om[0])
    pool = plan.alloc_pool(1)
    z = torch.empty(0, device="cuda:0")
    plan.step(pool, 0, z, z, z, z, z, z)
    torch.cuda.synchronize()
    assert int(pool.sum()) == 0

@pytest.mark.parametrize("kind,d,mode", [("kda", 128, 0), ("kda", 64, 0), ("kda", 128, 1),
                                         ("gdn", 128, 0), ("gdn", 64, 1)])
def test_decay_first_gate_order(torch_gpu, kind, d, mode):
    """Plan order 1, A = (I - beta k k^T) Diag(a): every tile and step against the oracle's
    decay-first step, fused and split, KDA with mixed rows and pivots and GDN with each width."""
    if kind == "kda":
        w = dataclasses.replace(_small(700 + d + mode, kind="kda", d=d, H=3), order=1)
        g = np.random.default_rng(d + mode)
        bits = g.choice([2, 4, 6, 8], size=(w.H, d)).astype(np.int8)
        piv = np.zeros((w.H, d), np.uint8)
        piv[1, g.choice(d, 5, replace=False)] = 1
        om = P.omega_from_steps(w, 0, "warmup", w.warmup)
    else:
        w = dataclasses.replace(_small(710 + d + mode, d=d, H=5, fixed_bits=(2, 4, 6, 8, 0)),
                                order=1)
        bits, piv, om = (a[0] for a in P.oracle_plan(w))
    P.log(f"[parity] decay-first {kind} d={d} mode={mode}")
    tr, plan, _ = P.run_layer(w, 0, bits, piv, om, w.steps, mode=mode)
    assert plan.status() == 0
